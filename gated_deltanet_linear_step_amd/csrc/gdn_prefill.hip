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
//                      Several sequences only: one sequence's chunk bounds are
//                      closed-form and the kernels below compute them.
//  2. prep_kernel   -- per (chunk, k-head), all chunks in parallel: q/k L2 norm,
//                      the gram K K^T and Q K^T (f16 MFMA, Q K^T from hi + lo
//                      parts), the normalised Q and K^T for the workspace; then for
//                      each v-head reading that k-head: gates and their in-chunk
//                      prefix sums, T = (I + A)^-1 in f32 (16x16 diagonal blocks by
//                      substitution, off-diagonal blocks by f32 MFMA block
//                      products), U and W (f16 MFMA), Aqk and the decay rows.
//  3. carry         -- per (sequence, v-head, 16-row slice of dv), sequential
//                      over the sequence's chunks: the slice's S^T stays in MFMA
//                      accumulators (f32), rounded to f16 as the B operand of
//                      W S^T and Q S^T; D enters the state update and the output
//                      as f16 hi + lo pairs. Two copy waves per workgroup bring
//                      each chunk's operands global -> LDS one chunk ahead.
//                      carry_split_kernel (few sequences: latency bound) gives
//                      each slice a compute wave for the recurrence and an output
//                      wave for O; carry_kernel (many sequences: throughput
//                      bound) does both in one wave per slice.
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

// Half offset of 16-byte block u (8 token slots) in row `row` of a transposed
// tile: the blocks are XOR-swizzled by row / 8. LDS serves 16-byte accesses
// eight lanes at a time over 32 banks. The pitch alone spreads the MFMA operand
// reads (eight consecutive rows, one block); the swizzle spreads the transposing
// stores (rows 4 dq + d for eight dq, one block), which the 144-byte pitch
// alone maps onto two bank groups.
__device__ __forceinline__ int tcol(int row, int u) { return 8 * (u ^ ((row >> 3) & 7)); }
constexpr int AP = C + 4;     // padded f32 row of the 64x64 A / T matrix

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
    size_t chunk_seq, chunk_start, chunk_len, seq_chunk0, seq_order, qn, knT, wmat, umat, aqk, gcum, onorm,
        total;
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
    L.seq_order = take(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    L.qn = take(sizeof(uint16_t) * MC * Hk * C * DH);
    L.knT = take(sizeof(uint16_t) * MC * Hk * DH * C);
    L.wmat = take(sizeof(uint16_t) * MC * Hv * C * DH);
    L.umat = take(sizeof(float) * MC * Hv * C * DH);
    L.aqk = take(sizeof(uint16_t) * MC * Hv * C * C);
    L.gcum = take(sizeof(float) * MC * Hv * 4 * C);
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
        const int len = i < p.N ? p.cu[i + 1] - p.cu[i] : 0;
        const int nc = (len + C - 1) / C;
        scan[threadIdx.x] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
            const int v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += v;
            __syncthreads();
        }
        if (i < p.N)
            p.seq_chunk0[i] = base_s + scan[threadIdx.x] - nc;
        // this block's chunks, one per thread: chunk c (counted from the block's
        // first) belongs to the first sequence whose inclusive count exceeds c
        const int total = scan[255];
        for (int c = threadIdx.x; c < total; c += 256) {
            int lo = 0, hi = 255;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (scan[mid] > c)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int k = c - (lo ? scan[lo - 1] : 0);  // chunk within its sequence
            const int seq = i0 + lo;
            const int s0 = p.cu[seq], sl = p.cu[seq + 1] - s0;
            const int g = base_s + c;
            p.chunk_seq[g] = seq;
            p.chunk_start[g] = s0 + k * C;
            p.chunk_len[g] = min(C, sl - k * C);
        }
        __syncthreads();
        if (threadIdx.x == 255)
            base_s += scan[255];
        __syncthreads();
    }
    // The carry takes sequences longest first (its workgroups are the sequential
    // chains; starting the long ones first shortens the whole call). Up to 256
    // sequences are ranked by chunk count (ties by index); more keep their order.
    if (p.N <= 256) {
        const int i = threadIdx.x;
        const int nc = i < p.N ? (p.cu[i + 1] - p.cu[i] + C - 1) / C : -1;
        scan[i] = nc;
        __syncthreads();
        if (i < p.N) {
            int rank = 0;
            for (int j = 0; j < p.N; ++j)
                rank += scan[j] > nc || (scan[j] == nc && j < i);
            p.seq_order[rank] = i;
        }
    } else {
        for (int i = threadIdx.x; i < p.N; i += 256)
            p.seq_order[i] = i;
    }
}

// ---------------------------------------------------------------- 2. prep

// One workgroup per (chunk, k-head): the normalised q/k rows, K K^T, Q K^T and
// the workspace's Q and K^T are formed once and serve the Hv/Hk v-heads that
// read this k-head, which the workgroup then takes in turn (gates, A and Aqk,
// the inverse, U and W, the decay rows).
template <int QT>
__global__ __launch_bounds__(256, 2) void prep_kernel(PrefillParams p)
{
    // LDS: X1 = normalised K rows (f16) then A / T (f32, in place, per v-head);
    //      X2 = normalised Q rows (f16), then per v-head the block-product
    //      scratch (f32) and W (f16, staged for the store).
    // K and Q rows are stored with dk in the permuted order, which W and Q keep.
    __shared__ __attribute__((aligned(16))) unsigned char X1[C * AP * 4];
    __shared__ __attribute__((aligned(16))) unsigned char X2[C * KP * 2];
    __shared__ __attribute__((aligned(16))) _Float16 VT[DH][TP];  // v, [dv][token slot] (per v-head)
    __shared__ __attribute__((aligned(16))) _Float16 KT[DH][TP];  // k, [dk slot][token slot]
    __shared__ __attribute__((aligned(16))) float G_s[C], beta_s[C], bg_s[C];
    static_assert(C * AP * 4 >= C * KP * 2, "X1 holds both the K rows and A / T");
    static_assert((AP * 4) % 16 == 0, "A / T rows are 16-byte aligned");
    static_assert(C * KP * 2 >= 32 * 36 * 4, "X2 holds the Q rows and the 32x32 scratch");

    _Float16(*Kh)[KP] = reinterpret_cast<_Float16(*)[KP]>(X1);
    _Float16(*Qh)[KP] = reinterpret_cast<_Float16(*)[KP]>(X2);
    // f16 remainders (x - f16(x)) of the normalised rows, for Q K^T; they live
    // in the transposed tiles' space, which is filled only after that product
    _Float16(*Kl)[KP] = reinterpret_cast<_Float16(*)[KP]>(&VT[0][0]);
    _Float16(*Ql)[KP] = reinterpret_cast<_Float16(*)[KP]>(&KT[0][0]);
    static_assert(sizeof(VT) >= C * KP * 2, "VT holds the K remainders");
    float(*Am)[AP] = reinterpret_cast<float(*)[AP]>(X1);
    float(*Pm)[36] = reinterpret_cast<float(*)[36]>(X2);
    // -scale Aqk (f16, token slots in the permuted order), staged behind Pm for a
    // coalesced copy to the workspace
    uint16_t(*Aqs)[C] = reinterpret_cast<uint16_t(*)[C]>(X2 + 32 * 36 * 4);
    static_assert(32 * 36 * 4 + C * C * 2 <= C * KP * 2, "X2 holds Pm and the staged Aqk");

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv, Hk = hc.Hk, G = Hv / Hk;
    const int chunk = blockIdx.x / Hk;
    const int kh = blockIdx.x % Hk;
    // one sequence covers tokens [0, total) (the host checks cu[0] = 0 and
    // cu[N] = total): its chunk bounds need no table, and no plan kernel runs
    const bool one_seq = p.N == 1;
    const int tok0 = one_seq ? C * chunk : p.chunk_start[chunk];
    const int n = one_seq ? min(C, p.total - C * chunk) : p.chunk_len[chunk];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const uint32_t flags = hc.flags;
    // the j-th v-head reading kh (the inverse of the head map)
    auto vhead = [&](int j) { return hc.head_map == 0 ? kh * G + j : kh + j * Hk; };
    // transposed tiles: thread = (four adjacent dims dq, token octet oc), the
    // octet being token slots 8 oc .. 8 oc + 7 of the permuted order
    const int dq = threadIdx.x & 31, oc = threadIdx.x >> 5;
    auto load_v = [&](Raw4<QT> (&vr)[8], int h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = perm_idx(8 * oc + i);
            vr[i] = load_raw4<QT>(in.v, (int64_t)(tok0 + min(t, n - 1)) * in.v_stride + (int64_t)h * DH + 4 * dq);
        }
    };

    // gate inputs of one v-head (wave 0, lane = token; lanes past the chunk's end
    // re-read its last token and are zeroed when used), fetched one v-head ahead
    const bool raw = flags & F_RAW_GATES;
    const void *gsrc_a = raw ? in.a : static_cast<const void *>(in.g);
    const void *gsrc_b = raw ? in.b : static_cast<const void *>(in.beta);
    const int gdt = raw ? in.ab_dt : DT_F32;
    GateWord ga, gb;
    float gdp = 0.f, gdb = 0.f;
    auto load_gates = [&](int h) {
        const int64_t gi = (int64_t)(tok0 + min(lane, n - 1)) * Hv + h;
        ga = load_gate(gsrc_a, gi, gdt);
        gb = load_gate(gsrc_b, gi, gdt);
        if (raw) {
            gdp = in.decay_param[h];
            gdb = in.dt_bias[h];
        }
    };
    if (wave == 0)
        load_gates(vhead(0));

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
            const float4 kz = make_float4(keep * kk.x, keep * kk.y, keep * kk.z, keep * kk.w);
            const float4 qz = make_float4(keep * qq.x, keep * qq.y, keep * qq.z, keep * qq.w);
            const half4 kh4 = {(_Float16)kz.x, (_Float16)kz.y, (_Float16)kz.z, (_Float16)kz.w};
            const half4 qh4 = {(_Float16)qz.x, (_Float16)qz.y, (_Float16)qz.z, (_Float16)qz.w};
            const half4 kl4 = {(_Float16)(kz.x - (float)kh4[0]), (_Float16)(kz.y - (float)kh4[1]),
                               (_Float16)(kz.z - (float)kh4[2]), (_Float16)(kz.w - (float)kh4[3])};
            const half4 ql4 = {(_Float16)(qz.x - (float)qh4[0]), (_Float16)(qz.y - (float)qh4[1]),
                               (_Float16)(qz.z - (float)qh4[2]), (_Float16)(qz.w - (float)qh4[3])};
            const int c4p = perm_pos(c4);  // the four stay adjacent
            *reinterpret_cast<half4 *>(&Kh[t][c4p]) = kh4;
            *reinterpret_cast<half4 *>(&Qh[t][c4p]) = qh4;
            *reinterpret_cast<half4 *>(&Kl[t][c4p]) = kl4;
            *reinterpret_cast<half4 *>(&Ql[t][c4p]) = ql4;
        }
    }
    __syncthreads();

    // the first v-head's v rows, in flight during the products below
    Raw4<QT> vr[8];
    load_v(vr, vhead(0));

    // -- K K^T and Q K^T on the lower block triangle: wave w owns token rows 16w..
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
                const half8 ql = lds_half8(&Ql[wave * 16 + li][ks * 32 + lg * 8]);
                const half8 kb = lds_half8(&Kh[j * 16 + li][ks * 32 + lg * 8]);
                const half8 kl = lds_half8(&Kl[j * 16 + li][ks * 32 + lg * 8]);
                gram[j] = mfma16(ka, kb, gram[j]);
                // Q K^T from hi + lo parts of both (the lo x lo term is below f32 rounding)
                qk[j] = mfma16(qa, kb, qk[j]);
                qk[j] = mfma16(qa, kl, qk[j]);
                qk[j] = mfma16(ql, kb, qk[j]);
            }
        }
    }

    __syncthreads();  // the remainders are dead: the transposed tiles take their space

    // -- K as [dk slot][token slot]; the K^T the carry reads ([dk][token slot], dk
    // natural) goes straight to the workspace from the same registers
    {
        typedef _Float16 half4 __attribute__((ext_vector_type(4)));
        half8 kt[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const half4 kq = *reinterpret_cast<const half4 *>(&Kh[perm_idx(8 * oc + i)][4 * dq]);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                kt[d][i] = kq[d];
        }
        uint16_t *kdst = p.knT + ((int64_t)chunk * Hk + kh) * DH * C;
        const int dk0 = perm_idx(4 * dq);  // slots 4dq .. 4dq+3 hold dk0 .. dk0+3
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            *reinterpret_cast<half8 *>(&KT[4 * dq + d][tcol(4 * dq + d, oc)]) = kt[d];
            *reinterpret_cast<half8 *>(kdst + (dk0 + d) * C + 8 * oc) = kt[d];
        }
    }
    // normalised Q rows (dk already in slot order) go to the workspace
    {
        uint16_t *qdst = p.qn + ((int64_t)chunk * Hk + kh) * C * DH;
#pragma unroll
        for (int k = 0; k < (C * DH / 8) / 256; ++k) {
            const int e = k * 256 + threadIdx.x;
            const int t = e / (DH / 8), c8 = (e % (DH / 8)) * 8;
            *reinterpret_cast<half8 *>(qdst + t * DH + c8) = lds_half8(&Qh[t][c8]);
        }
    }

    for (int j = 0; j < G; ++j) {
        const int h = vhead(j);
        // the previous v-head is done with LDS (W copied out, tiles read)
        __syncthreads();
        // -- gates and their prefix sums (wave 0, lane = token)
        if (wave == 0) {
            float g = gate_value(ga, gdt), beta = gate_value(gb, gdt);
            if (raw) {
                const float rate = hc.decay_kind == 0 ? -expf(gdp) : gdp;
                g = rate * softplus_f(g + gdb);
                beta = sigmoid_f(beta);
            }
            if (lane >= n)
                g = beta = 0.f;
            if (j + 1 < G)
                load_gates(vhead(j + 1));
            float Gc = g;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(Gc, off, 64);
                if (lane >= off)
                    Gc += o;
            }
            G_s[lane] = Gc;  // tokens >= n carry G_{n-1} (their g is 0)
            beta_s[lane] = beta;
            bg_s[lane] = beta * __expf(Gc);
        }
        // -- v as [dv][token slot]
        {
            half8 vb[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 vf = raw4_to_f32<QT>(vr[i]);
                vb[0][i] = (_Float16)vf.x;
                vb[1][i] = (_Float16)vf.y;
                vb[2][i] = (_Float16)vf.z;
                vb[3][i] = (_Float16)vf.w;
            }
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<half8 *>(&VT[4 * dq + d][tcol(4 * dq + d, oc)]) = vb[d];
        }
        if (j + 1 < G)
            load_v(vr, vhead(j + 1));  // the next v-head's rows, in flight from here
        __syncthreads();

        // -- A (strictly lower, f32) into X1; decayed, masked, scaled -Q K^T staged in X2
        {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = wave * 16 + lg * 4 + r, s = jj * 16 + li;
                    const float dg = s <= t ? __expf(G_s[t] - G_s[s]) : 0.f;
                    Am[t][s] = s < t ? beta_s[t] * dg * gram[jj][r] : 0.f;
                    Aqs[t][perm_pos(s)] = f32_to_f16_bits(-hc.scale * dg * qk[jj][r]);
                }
            }
        }
        __syncthreads();

        // -- T = (I + A)^-1 in place. (a) the four 16x16 diagonal blocks by forward
        // substitution: wave 0, lane = (block, column); meanwhile waves 1-3 copy
        // the staged -scale Aqk to the workspace.
        if (wave > 0) {
            uint16_t *aq = p.aqk + ((int64_t)chunk * Hv + h) * C * C;
            for (int e = threadIdx.x - 64; e < C * C / 8; e += 192) {
                const int t = e / (C / 8), c8 = (e % (C / 8)) * 8;
                *reinterpret_cast<uint4 *>(aq + t * C + c8) = *reinterpret_cast<const uint4 *>(&Aqs[t][c8]);
            }
        }
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

        // -- U = T diag(beta) V and W = T diag(beta gamma) K: wave w owns token rows
        // 16w..; the contraction runs over token slots, so T's columns are taken in
        // slot order, each scaled by its token's beta (U) or beta gamma (W)
        {
            // slots ks*32 + 8lg .. +7 are tokens ks*32 + 4lg .. +3 and ks*32 + 16 + 4lg .. +3:
            // two runs of four, read as 16-byte vectors
            half8 tu[2], tw[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int s0 = ks * 32 + 16 * hf + 4 * lg;
                    const f32x4 tv = *reinterpret_cast<const f32x4 *>(&Am[wave * 16 + li][s0]);
                    const f32x4 bt = *reinterpret_cast<const f32x4 *>(&beta_s[s0]);
                    const f32x4 bg = *reinterpret_cast<const f32x4 *>(&bg_s[s0]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tu[ks][4 * hf + i] = (_Float16)(tv[i] * bt[i]);
                        tw[ks][4 * hf + i] = (_Float16)(tv[i] * bg[i]);
                    }
                }
            float *ud = p.umat + ((int64_t)chunk * Hv + h) * DH * C;
            _Float16(*Wl)[KP] = reinterpret_cast<_Float16(*)[KP]>(X2);  // W rows, staged
#pragma unroll
            for (int nt = 0; nt < DH / 16; ++nt) {
                f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    u = mfma16(tu[ks], lds_half8(&VT[nt * 16 + li][tcol(nt * 16 + li, 4 * ks + lg)]), u);
                    w = mfma16(tw[ks], lds_half8(&KT[nt * 16 + li][tcol(nt * 16 + li, 4 * ks + lg)]), w);
                }
                // -U^T: this lane's four tokens are adjacent in row dv
                *reinterpret_cast<f32x4 *>(ud + (nt * 16 + li) * C + wave * 16 + lg * 4) = -u;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Wl[wave * 16 + lg * 4 + r][nt * 16 + li] = (_Float16)w[r];
            }
        }
        if (threadIdx.x < C) {
            // decay rows the carry multiplies by: gamma_t = exp(G_t),
            // -exp(G_last - G_t) (negated because the carry holds -D) and
            // scale gamma_t; G_last = G at the chunk's last token = G_s[C-1]
            float *gd = p.gcum + ((int64_t)chunk * Hv + h) * 4 * C;
            const float gm = __expf(G_s[threadIdx.x]);
            gd[threadIdx.x] = gm;
            gd[C + threadIdx.x] = -__expf(G_s[C - 1] - G_s[threadIdx.x]);
            gd[2 * C + threadIdx.x] = hc.scale * gm;
            gd[3 * C + threadIdx.x] = 0.f;
        }
        __syncthreads();
        {
            uint16_t *wd = p.wmat + ((int64_t)chunk * Hv + h) * C * DH;
            _Float16(*Wl)[KP] = reinterpret_cast<_Float16(*)[KP]>(X2);
#pragma unroll
            for (int k = 0; k < (C * DH / 8) / 256; ++k) {
                const int e = k * 256 + threadIdx.x;
                const int t = e / (DH / 8), c8 = (e % (DH / 8)) * 8;
                *reinterpret_cast<half8 *>(wd + t * DH + c8) = lds_half8(&Wl[t][c8]);
            }
        }
    }
}

// ---------------------------------------------------------------- 3. carry

// OUT: the output's dtype, or kOutNorm for the f32 buffer the gated norm reads
constexpr int kOutNorm = 3;

// LDS image of one chunk's operands for a workgroup covering NU 16-row dv
// slices. Rows are stored with their 16-byte blocks XOR-swizzled so that the 16
// rows one MFMA operand read touches fall in distinct banks: 256-byte rows (W, Q,
// -U^T) use block ^ (row & 15), 128-byte rows (K^T, Aqk) block ^ ((row >> 1) & 7).
template <int NU>
struct ChunkImage {
    unsigned char w[C * DH * 2];      // W   [t][dk (permuted)]        f16
    unsigned char q[C * DH * 2];      // Q   [t][dk (permuted)]        f16
    unsigned char kt[DH * C * 2];     // K^T [dk][t (permuted)]        f16
    unsigned char aq[C * C * 2];      // -scale Aqk [t][s (permuted)]  f16
    unsigned char u[16 * NU * C * 4]; // -U^T [dv - dvw][t]            f32
    float gd[4 * C];                  // decay rows, as the prep writes them
};

typedef __attribute__((address_space(3))) void lds_void;

// One asynchronous 16-byte-per-lane global -> LDS copy: lane l's bytes land at
// dst + 16 l (dst must be wave-uniform).
__device__ __forceinline__ void dma16(const unsigned char *src, unsigned char *dst)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, 0);
}

// Per-lane byte offsets of the global blocks a lane copies; they depend on the
// lane and the piece only, not on the chunk.
template <int NW, int NU>
struct CopyOffsets {
    uint32_t row256[16 / NW], row128[16 / NW], aq[8 / NW], u[(4 * NU) / NW];
};

template <int NW, int NU>
__device__ __forceinline__ CopyOffsets<NW, NU> copy_offsets(int wave, int lane)
{
    CopyOffsets<NW, NU> o;
    const int r256 = lane >> 4, s256 = lane & 15, r128 = lane >> 3, s128 = lane & 7;
#pragma unroll
    for (int k = 0; k < 16 / NW; ++k) {
        const int q = k * NW + wave;
        const int row = 4 * q + r256, krow = 8 * q + r128;
        o.row256[k] = row * 256 + 16 * (s256 ^ (row & 15));
        o.row128[k] = krow * 128 + 16 * (s128 ^ ((krow >> 1) & 7));
    }
#pragma unroll
    for (int k = 0; k < 8 / NW; ++k) {
        const int row = 8 * (k * NW + wave) + r128;
        o.aq[k] = row * 128 + 16 * (s128 ^ ((row >> 1) & 7));
    }
#pragma unroll
    for (int k = 0; k < (4 * NU) / NW; ++k) {
        const int row = 4 * (k * NW + wave) + r256;
        o.u[k] = row * 256 + 16 * (s256 ^ (row & 15));
    }
    return o;
}

// Issue the asynchronous global -> LDS copies of one chunk's operands; the NW
// waves of the workgroup split the one-KiB pieces between them (wave must be
// wave-uniform: it selects the LDS destination).
template <int NW, int NU>
__device__ __forceinline__ void issue_chunk_copy(ChunkImage<NU> &img, const PrefillParams &p,
                                                 const CopyOffsets<NW, NU> &o, int chunk, int h, int kh,
                                                 int dvw, int wave, int lane)
{
    const int Hv = p.hc.Hv, Hk = p.hc.Hk;
    const unsigned char *wg = reinterpret_cast<const unsigned char *>(p.wmat + ((int64_t)chunk * Hv + h) * C * DH);
    const unsigned char *qg = reinterpret_cast<const unsigned char *>(p.qn + ((int64_t)chunk * Hk + kh) * C * DH);
    const unsigned char *kg = reinterpret_cast<const unsigned char *>(p.knT + ((int64_t)chunk * Hk + kh) * DH * C);
    const unsigned char *ag = reinterpret_cast<const unsigned char *>(p.aqk + ((int64_t)chunk * Hv + h) * C * C);
    const unsigned char *ug = reinterpret_cast<const unsigned char *>(p.umat + (((int64_t)chunk * Hv + h) * DH + dvw) * C);
    static_assert(16 % NW == 0 && 8 % NW == 0 && (4 * NU) % NW == 0, "pieces split evenly");
#pragma unroll
    for (int k = 0; k < 16 / NW; ++k) {
        const int q = k * NW + wave;
        dma16(wg + o.row256[k], img.w + q * 1024);
        dma16(qg + o.row256[k], img.q + q * 1024);
        dma16(kg + o.row128[k], img.kt + q * 1024);
    }
#pragma unroll
    for (int k = 0; k < 8 / NW; ++k)
        dma16(ag + o.aq[k], img.aq + (k * NW + wave) * 1024);
#pragma unroll
    for (int k = 0; k < (4 * NU) / NW; ++k)
        dma16(ug + o.u[k], img.u + (k * NW + wave) * 1024);
    if (wave == 0) {  // the 1 KiB of decay rows
        const unsigned char *gg = reinterpret_cast<const unsigned char *>(p.gcum + ((int64_t)chunk * Hv + h) * 4 * C);
        dma16(gg + 16 * lane, reinterpret_cast<unsigned char *>(img.gd));
    }
}

__device__ __forceinline__ half8 img_half8(const unsigned char *base, int off)
{
    return *reinterpret_cast<const half8 *>(base + off);
}
__device__ __forceinline__ f32x4 img_f32x4(const unsigned char *base, int off)
{
    return *reinterpret_cast<const f32x4 *>(base + off);
}

// Two 16x16 accumulator tiles (rows r and r + 16 of a 32-block) as the eight
// f16 k-values one lane supplies to a 16x16x32 product, in the permuted order.
__device__ __forceinline__ half8 pack_tiles(const f32x4 &lo, const f32x4 &hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = __builtin_convertvector((f2){lo[0], lo[1]}, h2);
    const h2 b = __builtin_convertvector((f2){lo[2], lo[3]}, h2);
    const h2 c = __builtin_convertvector((f2){hi[0], hi[1]}, h2);
    const h2 d = __builtin_convertvector((f2){hi[2], hi[3]}, h2);
    return (half8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int V>
struct Slot {
    static constexpr int value = V;
};

// One output element through a buffer resource (offset in bytes).
template <int OUT>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x)
{
    if constexpr (OUT == DT_F32 || OUT == kOutNorm) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
    } else {
        // round to nearest even in hardware (v_cvt_pk_{bf16,f16}_f32)
        uint16_t v;
        if constexpr (OUT == DT_BF16) {
            const __bf16 b = (__bf16)x;
            __builtin_memcpy(&v, &b, 2);
        } else {
            v = f32_to_f16_bits(x);
        }
        __builtin_amdgcn_raw_buffer_store_b16(v, rs, off, 0, 0);
    }
}

// Output rows of one chunk (n valid tokens from token tok0). A full chunk
// stores without branches; a partial one masks the padding rows. The buffer
// resource's extent ends at the chunk's last valid row either way.
template <int OUT>
__device__ __forceinline__ void store_rows(const PrefillParams &p, int tok0, int n, int h, int64_t orow,
                                           uint32_t lane_off, int lg, const f32x4 (&O)[4])
{
    constexpr int ES = OUT == DT_F32 || OUT == kOutNorm ? 4 : 2;
    void *base = OUT == kOutNorm ? static_cast<void *>(p.onorm) : p.out;
    unsigned char *b = static_cast<unsigned char *>(base) + ((int64_t)tok0 * orow + (int64_t)h * DH) * ES;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)(n * orow * ES), 0x00020000);
    const uint32_t rstride = (uint32_t)(orow * ES);  // bytes per token row
    if (n == C) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_elem<OUT>(rs, lane_off + (16 * j + r) * rstride, O[j][r]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * j + 4 * lg + r < n)
                    store_elem<OUT>(rs, lane_off + (16 * j + r) * rstride, O[j][r]);
    }
}

// Carry: sequential over a sequence's chunks, one wave per 16-row slice of dv,
// NW slices (of one v-head) per workgroup. Wave state: S^T[dk][dv] for its 16
// dv columns in eight 16x16 f32 accumulator tiles, which also serve directly
// (rounded to f16) as the B operand of W S^T and Q S^T, so the chain from one
// chunk's state to the next never leaves the wave:
//   P' = W S^T - U  (= -D)                      accumulator seeded with -U
//   O  = scale gamma Q S^T + (-scale Aqk)(-D)      -D as an f16 hi + lo pair
//   S^T <- gamma_last S^T + K^T (D e)           D e as an f16 hi + lo pair
// with e_t = exp(G_last - G_t). The chunk's operands arrive in LDS through
// asynchronous global->LDS copies that two copy waves issue one chunk ahead
// into a two-slot ring (so the compute waves never stall behind a burst of
// vector-memory issues); outputs are stored one chunk late. One barrier per
// chunk.
template <int NW, int OUT>
__global__ __launch_bounds__(64 * (NW + 2), 1) void carry_kernel(PrefillParams p)
{
    __shared__ __attribute__((aligned(16))) ChunkImage<NW> img[2];

    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv;
    constexpr int NG = DH / (16 * NW);  // workgroups per (sequence, v-head)
    // XCD-aware order: the NG workgroups of one (sequence, head) share id % 8
    const int id = blockIdx.x;
    const int group = (id & 7) + 8 * (id / (8 * NG));
    const int part = (id >> 3) % NG;
    if (group >= p.N * Hv)
        return;
    const bool one_seq = p.N == 1;  // tokens [0, total), no tables (see prep_kernel)
    const int seq = one_seq ? 0 : p.seq_order[group / Hv], h = group % Hv;
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int dvw = part * 16 * NW;  // the workgroup's first dv row
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int dvl = dvw + wave * 16 + li;  // this lane's dv row
    const int start = one_seq ? 0 : p.cu[seq];
    const int len = one_seq ? p.total : p.cu[seq + 1] - start;
    const int nch = (len + C - 1) / C;
    if (nch == 0)
        return;  // empty sequence: state untouched
    const int c0 = one_seq ? 0 : p.seq_chunk0[seq];

    if (wave >= NW) {
        // copy waves: every chunk's operands, one chunk ahead, into the ring
        const int cw = wave - NW;
        const CopyOffsets<2, NW> co = copy_offsets<2, NW>(cw, lane);
        issue_chunk_copy<2, NW>(img[0], p, co, c0, h, kh, dvw, cw, lane);
        for (int ci = 0; ci < nch; ++ci) {
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): chunk ci has landed
            __builtin_amdgcn_s_barrier();
            if (ci + 1 < nch)
                issue_chunk_copy<2, NW>(img[(ci + 1) & 1], p, co, c0 + ci + 1, h, kh, dvw, cw, lane);
        }
        return;
    }

    // ST[m][r] = S[dvl][16m + 4lg + r]
    float *Sg = p.state + (((int64_t)seq * Hv + h) * DH + dvl) * DH + 4 * lg;
    f32x4 ST[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        ST[m] = *reinterpret_cast<const f32x4 *>(Sg + 16 * m);

    // per-lane byte offsets of the swizzled operand reads
    int wq[4], ka[2], uo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        wq[ks] = li * 256 + 16 * ((4 * ks + lg) ^ li);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        ka[ks] = li * 128 + 16 * ((4 * ks + lg) ^ ((li >> 1) & 7));
#pragma unroll
    for (int j = 0; j < 4; ++j)
        uo[j] = (wave * 16 + li) * 256 + 16 * ((4 * j + lg) ^ li);

    const int64_t orow = (int64_t)Hv * DH;
    constexpr int ES = OUT == DT_F32 || OUT == kOutNorm ? 4 : 2;
    const uint32_t lane_off = (uint32_t)((4 * lg * orow + dvl) * ES);
    f32x4 Oprev[4];
    int prev_tok0 = 0, prev_n = 0;

    auto step = [&](auto slot, int ci) {
        constexpr int SL = decltype(slot)::value;
        // this chunk's copies (issued one chunk ago) have landed, and every wave
        // is done reading the slot the next copies overwrite
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (ci > 0)
            store_rows<OUT>(p, prev_tok0, prev_n, h, orow, lane_off, lg, Oprev);
        const ChunkImage<NW> &cur = img[SL];
        // The phases below are kept in source order (scheduling fences) so that
        // each phase's LDS operand reads are in flight during the previous
        // phase's products instead of being issued just before their use.

        // phase 1: operands of P' = W S^T - U, decay rows; the state as B operand
        half8 wa[4][4];
        f32x4 Pn[4], er[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Pn[j] = img_f32x4(cur.u, uo[j]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                wa[j][ks] = img_half8(cur.w, wq[ks] + j * 4096);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            er[j] = *reinterpret_cast<const f32x4 *>(&cur.gd[C + 16 * j + 4 * lg]);
        // gamma_last = gamma_{C-1} (tokens past a short chunk carry G_{n-1}): one
        // broadcast LDS read. Taking it from lane 48's copy of a 16-byte row read
        // (readlane of element 3) was compiled into a read of element 0, gamma_{C-4}.
        const float gl = cur.gd[C - 1];
        half8 sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            sb[ks] = pack_tiles(ST[2 * ks], ST[2 * ks + 1]);
        __builtin_amdgcn_sched_barrier(0);

        // phase 2: P' products (consecutive ones into different accumulators),
        // with the state update's K^T operands read behind them
        half8 kb[8][2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = i & 3, ks = i >> 2;
            Pn[j] = mfma16(wa[j][ks], sb[ks], Pn[j]);
            kb[i >> 1][i & 1] = img_half8(cur.kt, ka[i & 1] + (i >> 1) * 2048);
            __builtin_amdgcn_sched_barrier(0);
        }

        // phase 3: -D as hi + lo (for the output), D e as hi + lo (for the state)
        half8 dn[2], dnl[2], dh[2], dl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const f32x4 a = Pn[2 * ks] * er[2 * ks], b = Pn[2 * ks + 1] * er[2 * ks + 1];
            dn[ks] = pack_tiles(Pn[2 * ks], Pn[2 * ks + 1]);
            dh[ks] = pack_tiles(a, b);
            f32x4 ar, br, pr, qr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ar[i] = a[i] - (float)dh[ks][i];
                br[i] = b[i] - (float)dh[ks][4 + i];
                pr[i] = Pn[2 * ks][i] - (float)dn[ks][i];
                qr[i] = Pn[2 * ks + 1][i] - (float)dn[ks][4 + i];
            }
            dl[ks] = pack_tiles(ar, br);
            dnl[ks] = pack_tiles(pr, qr);
        }
        __builtin_amdgcn_sched_barrier(0);

        // phase 4: S^T <- gamma_last S^T + K^T (D e), with the output's operands read behind
        half8 qa[4][4], aa[6];
        f32x4 gm[4];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            ST[m] *= gl;
#pragma unroll
        for (int i2 = 0; i2 < 32; ++i2) {
            const int m = i2 & 7, ks = i2 >> 4;
            ST[m] = mfma16(kb[m][ks], (i2 >> 3) & 1 ? dl[ks] : dh[ks], ST[m]);
            if (i2 & 1) {
                const int i = i2 >> 1;  // 16 Q reads, then Aqk and the gamma rows
                qa[i >> 2][i & 3] = img_half8(cur.q, wq[i & 3] + (i >> 2) * 4096);
                if (i < 6)
                    aa[i] = img_half8(cur.aq, ka[i < 2 ? 0 : (i & 1)] + (i < 2 ? i : (i + 2) >> 1) * 2048);
                if (i >= 6 && i < 10)
                    gm[i - 6] = *reinterpret_cast<const f32x4 *>(&cur.gd[2 * C + 16 * (i - 6) + 4 * lg]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // phase 5: O = scale gamma Q S^T + (-scale Aqk)(-D), off the state's chain
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qs = mfma16(qa[j][ks], sb[ks], qs);
            qs *= gm[j];
            // Aqk tiles (j, ks) with ks <= j / 2, in aa order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (2 * ks <= j) {
                    const half8 &a = aa[j < 2 ? j : 2 + 2 * (j - 2) + ks];
                    qs = mfma16(a, dn[ks], qs);
                    qs = mfma16(a, dnl[ks], qs);
                }
            Oprev[j] = qs;
        }
        prev_tok0 = start + ci * C;
        prev_n = min(C, len - ci * C);
    };

    for (int ci = 0; ci < nch; ci += 2) {
        step(Slot<0>{}, ci);
        if (ci + 1 < nch)
            step(Slot<1>{}, ci + 1);
    }
    store_rows<OUT>(p, prev_tok0, prev_n, h, orow, lane_off, lg, Oprev);
#pragma unroll
    for (int m = 0; m < 8; ++m)
        *reinterpret_cast<f32x4 *>(Sg + 16 * m) = ST[m];
}

// Carry with the output products moved off the state's chain. Per 16-row dv
// slice a compute wave runs the recurrence (P' = W S^T - U, D, S^T update) and
// an output wave forms O = scale gamma Q S^T + (-scale Aqk)(-D) from the
// state and -D the compute wave leaves in LDS; two copy waves keep the operand
// ring one chunk ahead. Two barriers per chunk: A (chunk landed, state
// published) and B (-D published).
template <int NW, int OUT>
__global__ __launch_bounds__(64 * (2 * NW + 2), 1) void carry_split_kernel(PrefillParams p)
{
    __shared__ __attribute__((aligned(16))) ChunkImage<NW> img[2];
    // per slice: [0..3] S^T as the f16 B operand, [4..5] -D hi, [6..7] -D lo
    __shared__ __attribute__((aligned(16))) half8 xs[NW][8][64];

    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv;
    constexpr int NG = DH / (16 * NW);
    const int id = blockIdx.x;
    const int group = (id & 7) + 8 * (id / (8 * NG));
    const int part = (id >> 3) % NG;
    if (group >= p.N * Hv)
        return;
    const bool one_seq = p.N == 1;  // tokens [0, total), no tables (see prep_kernel)
    const int seq = one_seq ? 0 : p.seq_order[group / Hv], h = group % Hv;
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int dvw = part * 16 * NW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int start = one_seq ? 0 : p.cu[seq];
    const int len = one_seq ? p.total : p.cu[seq + 1] - start;
    const int nch = (len + C - 1) / C;
    if (nch == 0)
        return;
    const int c0 = one_seq ? 0 : p.seq_chunk0[seq];

    if (wave >= 2 * NW) {
        const int cw = wave - 2 * NW;
        const CopyOffsets<2, NW> co = copy_offsets<2, NW>(cw, lane);
        issue_chunk_copy<2, NW>(img[0], p, co, c0, h, kh, dvw, cw, lane);
        for (int ci = 0; ci < nch; ++ci) {
            __builtin_amdgcn_s_waitcnt(0x0070);  // chunk ci has landed
            __builtin_amdgcn_s_barrier();        // A
            if (ci + 1 < nch)
                issue_chunk_copy<2, NW>(img[(ci + 1) & 1], p, co, c0 + ci + 1, h, kh, dvw, cw, lane);
            __builtin_amdgcn_s_barrier();        // B
        }
        return;
    }

    const int sl = wave < NW ? wave : wave - NW;  // slice within the workgroup
    const int dvl = dvw + sl * 16 + li;
    int wq[4], ka[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        wq[ks] = li * 256 + 16 * ((4 * ks + lg) ^ li);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        ka[ks] = li * 128 + 16 * ((4 * ks + lg) ^ ((li >> 1) & 7));
    half8 *xw = &xs[sl][0][lane];  // xw[64 * i] is entry i of this lane

    if (wave < NW) {
        // ---- compute wave
        float *Sg = p.state + (((int64_t)seq * Hv + h) * DH + dvl) * DH + 4 * lg;
        f32x4 ST[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            ST[m] = *reinterpret_cast<const f32x4 *>(Sg + 16 * m);
        int uo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            uo[j] = (sl * 16 + li) * 256 + 16 * ((4 * j + lg) ^ li);
        half8 sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            sb[ks] = pack_tiles(ST[2 * ks], ST[2 * ks + 1]);
            xw[64 * ks] = sb[ks];
        }

        auto step = [&](auto slot) {
            constexpr int SL = decltype(slot)::value;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the state is published
            __builtin_amdgcn_s_barrier();        // A
            const ChunkImage<NW> &cur = img[SL];
            half8 wa[4][4];
            f32x4 Pn[4], er[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Pn[j] = img_f32x4(cur.u, uo[j]);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    wa[j][ks] = img_half8(cur.w, wq[ks] + j * 4096);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                er[j] = *reinterpret_cast<const f32x4 *>(&cur.gd[C + 16 * j + 4 * lg]);
            const float gl = cur.gd[C - 1];  // gamma_last, a broadcast read (see carry_kernel)
            __builtin_amdgcn_sched_barrier(0);

            half8 kb[8][2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = i & 3, ks = i >> 2;
                Pn[j] = mfma16(wa[j][ks], sb[ks], Pn[j]);
                kb[i >> 1][i & 1] = img_half8(cur.kt, ka[i & 1] + (i >> 1) * 2048);
                __builtin_amdgcn_sched_barrier(0);
            }

            half8 dh[2], dl[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 a = Pn[2 * ks] * er[2 * ks], b = Pn[2 * ks + 1] * er[2 * ks + 1];
                const half8 dn = pack_tiles(Pn[2 * ks], Pn[2 * ks + 1]);
                dh[ks] = pack_tiles(a, b);
                f32x4 ar, br, pr, qr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ar[i] = a[i] - (float)dh[ks][i];
                    br[i] = b[i] - (float)dh[ks][4 + i];
                    pr[i] = Pn[2 * ks][i] - (float)dn[i];
                    qr[i] = Pn[2 * ks + 1][i] - (float)dn[4 + i];
                }
                dl[ks] = pack_tiles(ar, br);
                xw[64 * (4 + ks)] = dn;
                xw[64 * (6 + ks)] = pack_tiles(pr, qr);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): -D is published
            __builtin_amdgcn_s_barrier();        // B

#pragma unroll
            for (int m = 0; m < 8; ++m)
                ST[m] *= gl;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int m = i & 7, ks = i >> 4;
                ST[m] = mfma16(kb[m][ks], (i >> 3) & 1 ? dl[ks] : dh[ks], ST[m]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                sb[ks] = pack_tiles(ST[2 * ks], ST[2 * ks + 1]);
                xw[64 * ks] = sb[ks];
            }
        };
        for (int ci = 0; ci < nch; ci += 2) {
            step(Slot<0>{});
            if (ci + 1 < nch)
                step(Slot<1>{});
        }
#pragma unroll
        for (int m = 0; m < 8; ++m)
            *reinterpret_cast<f32x4 *>(Sg + 16 * m) = ST[m];
        return;
    }

    // ---- output wave
    const int64_t orow = (int64_t)Hv * DH;
    constexpr int ES = OUT == DT_F32 || OUT == kOutNorm ? 4 : 2;
    const uint32_t lane_off = (uint32_t)((4 * lg * orow + dvl) * ES);
    auto ostep = [&](auto slot, int ci) {
        constexpr int SL = decltype(slot)::value;
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();  // A
        const ChunkImage<NW> &cur = img[SL];
        half8 sbr[4], qa[4][4], aa[6];
        f32x4 gm[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            sbr[ks] = xw[64 * ks];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            qa[i & 3][i >> 2] = img_half8(cur.q, wq[i >> 2] + (i & 3) * 4096);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            gm[j] = *reinterpret_cast<const f32x4 *>(&cur.gd[2 * C + 16 * j + 4 * lg]);
#pragma unroll
        for (int i = 0; i < 6; ++i)
            aa[i] = img_half8(cur.aq, ka[i < 2 ? 0 : (i & 1)] + (i < 2 ? i : (i + 2) >> 1) * 2048);
        f32x4 qs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qs[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = i & 3, ks = i >> 2;
            qs[j] = mfma16(qa[j][ks], sbr[ks], qs[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qs[j] *= gm[j];
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();  // B
        half8 dn[2], dnl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            dn[ks] = xw[64 * (4 + ks)];
            dnl[ks] = xw[64 * (6 + ks)];
        }
        // Aqk tiles (j, ks) with ks <= j / 2, in aa order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
        for (int part2 = 0; part2 < 2; ++part2)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (2 * ks <= j)
                        qs[j] = mfma16(aa[j < 2 ? j : 2 + 2 * (j - 2) + ks], part2 ? dnl[ks] : dn[ks], qs[j]);
        store_rows<OUT>(p, start + ci * C, min(C, len - ci * C), h, orow, lane_off, lg, qs);
    };
    for (int ci = 0; ci < nch; ci += 2) {
        ostep(Slot<0>{}, ci);
        if (ci + 1 < nch)
            ostep(Slot<1>{}, ci + 1);
    }
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

// 128 x 128 runs the f16-operand MFMA kernels of this file; the decode's other
// head shapes run the f32-accuracy path of gdn_prefill_generic.hip.
bool prefill_supported(int dk, int dv) { return (dk == DH && dv == DH) || prefill_generic_supported(dk, dv); }

bool prefill_is_mfma(int dk, int dv) { return dk == DH && dv == DH; }

int prefill_chunk_len(int dk, int dv) { return prefill_is_mfma(dk, dv) ? C : prefill_generic_chunk(dk); }

// max_chunks bounds the chunk count of the call (total / chunk length + N).
size_t prefill_workspace_bytes(int Hk, int Hv, int dk, int dv, int64_t max_chunks, int N,
                               int64_t total_tokens, bool norm)
{
    if (!prefill_is_mfma(dk, dv))
        return prefill_generic_workspace_bytes(Hk, Hv, dk, dv, max_chunks, N, total_tokens, norm);
    return ws_layout(Hk, Hv, max_chunks, N, total_tokens, norm).total;
}

void prefill_carve(PrefillParams &p, void *ws, int64_t max_chunks)
{
    if (!prefill_is_mfma(p.hc.dk, p.hc.dv)) {
        prefill_generic_carve(p, ws, max_chunks);
        return;
    }
    const WsLayout L = ws_layout(p.hc.Hk, p.hc.Hv, max_chunks, p.N, p.total,
                                 (p.hc.flags & F_GATED_NORM) != 0);
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.chunk_seq = reinterpret_cast<int32_t *>(b + L.chunk_seq);
    p.chunk_start = reinterpret_cast<int32_t *>(b + L.chunk_start);
    p.chunk_len = reinterpret_cast<int32_t *>(b + L.chunk_len);
    p.seq_chunk0 = reinterpret_cast<int32_t *>(b + L.seq_chunk0);
    p.seq_order = reinterpret_cast<int32_t *>(b + L.seq_order);
    p.qn = reinterpret_cast<uint16_t *>(b + L.qn);
    p.knT = reinterpret_cast<uint16_t *>(b + L.knT);
    p.wmat = reinterpret_cast<uint16_t *>(b + L.wmat);
    p.umat = reinterpret_cast<float *>(b + L.umat);
    p.aqk = reinterpret_cast<uint16_t *>(b + L.aqk);
    p.gcum = reinterpret_cast<float *>(b + L.gcum);
    p.onorm = reinterpret_cast<float *>(b + L.onorm);
}

template <int NW>
void launch_carry_split(const PrefillParams &p, const PrefillPlan &pl, hipStream_t s)
{
    const dim3 cgrid((unsigned)pl.carry_workgroups);
    const dim3 cblock(64 * (2 * NW + 2));
    const int omode = (p.hc.flags & F_GATED_NORM) ? kOutNorm : p.out_dt;
    switch (omode) {
    case kOutNorm: hipLaunchKernelGGL((carry_split_kernel<NW, kOutNorm>), cgrid, cblock, 0, s, p); break;
    case DT_F32: hipLaunchKernelGGL((carry_split_kernel<NW, DT_F32>), cgrid, cblock, 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((carry_split_kernel<NW, DT_F16>), cgrid, cblock, 0, s, p); break;
    default: hipLaunchKernelGGL((carry_split_kernel<NW, DT_BF16>), cgrid, cblock, 0, s, p); break;
    }
}

template <int NW>
void launch_carry(const PrefillParams &p, const PrefillPlan &pl, hipStream_t s)
{
    const dim3 cgrid((unsigned)pl.carry_workgroups);
    const dim3 cblock(64 * (NW + 2));
    const int omode = (p.hc.flags & F_GATED_NORM) ? kOutNorm : p.out_dt;
    switch (omode) {
    case kOutNorm: hipLaunchKernelGGL((carry_kernel<NW, kOutNorm>), cgrid, cblock, 0, s, p); break;
    case DT_F32: hipLaunchKernelGGL((carry_kernel<NW, DT_F32>), cgrid, cblock, 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((carry_kernel<NW, DT_F16>), cgrid, cblock, 0, s, p); break;
    default: hipLaunchKernelGGL((carry_kernel<NW, DT_BF16>), cgrid, cblock, 0, s, p); break;
    }
}

// Carry shape (each workgroup takes a whole CU's LDS): while one round of
// workgroups covers every dv slice the call is bound by the per-chunk chain, so
// the split carry runs with 1 slice per workgroup (8 per head) or, when that would
// take two rounds, 2; beyond that it is throughput bound and the 4-slice carry,
// which reads each chunk's shared operands once for 4 slices, is fastest.
PrefillPlan prefill_plan(int N, int Hk, int Hv, int dk, int dv, int64_t num_chunks, int cus)
{
    PrefillPlan pl{};
    if (!prefill_supported(dk, dv))
        return pl;
    if (!prefill_is_mfma(dk, dv)) {  // f32 path: carry per (sequence, v-head, 32 dv rows)
        pl.carry_kind = 2;
        pl.slices_per_wg = 2;
        pl.carry_workgroups = (int)((int64_t)N * Hv * (dv / 32));
        pl.carry_threads = prefill_generic_carry_threads();
        pl.prep_workgroups = (int)(num_chunks * Hk);
        return pl;
    }
    const int64_t groups = (int64_t)N * Hv;
    const int64_t rounded = (groups + 7) / 8 * 8;  // XCD-aware order: groups in blocks of 8
    if (groups * (DH / 16) <= cus) {
        pl.carry_kind = 0;
        pl.slices_per_wg = 1;
        pl.carry_threads = 64 * (2 * 1 + 2);
    } else if (groups * (DH / 32) <= cus) {
        pl.carry_kind = 0;
        pl.slices_per_wg = 2;
        pl.carry_threads = 64 * (2 * 2 + 2);
    } else {
        pl.carry_kind = 1;
        pl.slices_per_wg = 4;
        pl.carry_threads = 64 * (4 + 2);
    }
    pl.carry_workgroups = (int)(rounded * (DH / (16 * pl.slices_per_wg)));
    pl.prep_workgroups = (int)(num_chunks * Hk);
    return pl;
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s)
{
    if (p.num_chunks == 0)
        return hipSuccess;
    if (!prefill_is_mfma(p.hc.dk, p.hc.dv))
        return launch_prefill_generic(p, s);
    if (p.N > 1)  // one sequence: the chunk bounds are closed-form, no table
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    int cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const PrefillPlan pl = prefill_plan(p.N, p.hc.Hk, p.hc.Hv, p.hc.dk, p.hc.dv, p.num_chunks, cus);
    const dim3 pgrid((unsigned)pl.prep_workgroups);
    switch (p.in.qkv_dt) {
    case DT_F32: hipLaunchKernelGGL((prep_kernel<DT_F32>), pgrid, dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((prep_kernel<DT_F16>), pgrid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((prep_kernel<DT_BF16>), pgrid, dim3(256), 0, s, p); break;
    }
    if (pl.carry_kind == 0 && pl.slices_per_wg == 1)
        launch_carry_split<1>(p, pl, s);
    else if (pl.carry_kind == 0)
        launch_carry_split<2>(p, pl, s);
    else
        launch_carry<4>(p, pl, s);
    if (p.hc.flags & F_GATED_NORM) {
        const int64_t rows = (int64_t)p.total * p.hc.Hv;
        hipLaunchKernelGGL(norm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
