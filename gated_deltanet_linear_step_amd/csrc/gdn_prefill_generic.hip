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
// Kernels (f32 accuracy throughout: the preparation's products on
// v_mfma_f32_16x16x4_f32, the carry's on v_mfma_f32_16x16x32_bf16 with each f32
// operand split into a bf16 hi/lo pair):
//  1. plan_generic_kernel -- the chunk table (several sequences only; one
//     sequence's chunk bounds are closed-form).
//  2. prep_generic_kernel -- per (chunk, k-head), all chunks in parallel: the
//     normalised q and k rows, the lower triangles of K K^T and Q K^T once, then
//     for each v-head reading the k-head: gates and their prefix sums, A,
//     T = (I + A)^-1 (16 x 16 diagonal blocks by substitution, the blocks below
//     by block products), W, U, scale * Aqk, diag(e) K and the decay rows, all to
//     the workspace.
//  3. carry_generic_kernel -- per (sequence, v-head, 32 rows of dv), sequential
//     over the sequence's chunks with the slice's f32 state resident in MFMA
//     accumulators: only the state-dependent products (Q S^T, W S^T, Aqk D,
//     D^T diag(e) K). The next chunk's operands are loaded into registers while
//     the current one runs.
//  4. norm_generic_kernel -- the gated RMS norm of the f32 core output.
// Chunks are 64 tokens, 32 when dk = 256 (the LDS then holds the 256-wide tiles).
// LDS row pitches are chosen by how the MFMA operand reads index each array. The
// LDS serves a 32-bit read in two halves of 32 lanes over 32 banks, so an array
// whose row is the lane's m or n index (lane % 16, column lane / 16) takes a
// pitch of 2 mod 4 floats, and one whose row is the contracted index (lane / 16,
// column lane % 16) a pitch of 16 mod 32: both spread each half over 32 banks.

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kSlice = 32;  // dv rows per carry workgroup

template <int DK>
constexpr int gen_chunk()
{
    return DK >= 256 ? 32 : 64;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// x as a pair of bf16 (hi = x rounded to nearest even, lo = the rest rounded),
// hi + lo = x to about 2^-16 relative; a product of two such pairs taken as
// hi*hi + hi*lo + lo*hi on bf16 MFMA keeps that accuracy with f32 range.
__device__ __forceinline__ void bf16_split(float x, uint16_t &hi, uint16_t &lo)
{
    const __bf16 h = (__bf16)x;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)h));
}

// Element idx of a workspace array of n values stored as a [hi block][lo block]
// pair of bf16 arrays (4 bytes per value, as f32).
__device__ __forceinline__ void put_pair(float *base, int64_t n, int64_t idx, float x)
{
    uint16_t *b = reinterpret_cast<uint16_t *>(base);
    uint16_t h, l;
    bf16_split(x, h, l);
    b[idx] = h;
    b[n + idx] = l;
}

// One 16 x 16 tile of sum_k a(m, k) b(k, n) over k in [kb, kb + 4 KSTEPS) on
// v_mfma_f32_16x16x4_f32, as two accumulator chains (alternate k-steps) added at
// the end. Lane (li, lg) = (lane % 16, lane / 16) feeds a(m0 + li, k0 + lg) and
// b(k0 + lg, n0 + li) and receives C[m0 + 4 lg + r][n0 + li] in element r.
template <int KSTEPS, class FA, class FB>
__device__ __forceinline__ f32x4 mfma_tile(FA a, FB b, int m0, int n0, int kb = 0)
{
    static_assert(KSTEPS % 2 == 0, "two chains");
    // operands are read a block of BLK k-steps at a time, the next block's reads
    // issued before this block's products
    constexpr int BLK = KSTEPS % 8 == 0 ? 8 : KSTEPS;
    static_assert(KSTEPS % BLK == 0, "blocks");
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    float av[BLK], bv[BLK];
#pragma unroll
    for (int s = 0; s < BLK; ++s) {
        av[s] = a(m0 + li, kb + 4 * s + lg);
        bv[s] = b(kb + 4 * s + lg, n0 + li);
    }
    // keep the reads ahead of the products (the scheduler would otherwise sink
    // each read next to its use and wait on it)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int blk = 0; blk < KSTEPS; blk += BLK) {
        float an[BLK], bn[BLK];
        if (blk + BLK < KSTEPS) {
#pragma unroll
            for (int s = 0; s < BLK; ++s) {
                an[s] = a(m0 + li, kb + 4 * (blk + BLK + s) + lg);
                bn[s] = b(kb + 4 * (blk + BLK + s) + lg, n0 + li);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < BLK; s += 2) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s + 1], bv[s + 1], c1, 0, 0, 0);
        }
        if (blk + BLK < KSTEPS) {
#pragma unroll
            for (int s = 0; s < BLK; ++s) {
                av[s] = an[s];
                bv[s] = bn[s];
            }
        }
    }
    return c0 + c1;
}

// Two tiles that share the right operand, a1 b and a2 b over k in [kb, kb + 4
// KSTEPS): one read of b serves both products; reads go a block ahead as above.
template <int KSTEPS, class FA1, class FA2, class FB>
__device__ __forceinline__ void mfma_tile2(FA1 a1, FA2 a2, FB b, int m0, int n0, int kb, f32x4 &r1, f32x4 &r2)
{
    constexpr int BLK = KSTEPS < 8 ? KSTEPS : 8;
    static_assert(KSTEPS % BLK == 0 && BLK % 2 == 0, "blocks");
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, d0 = c0, d1 = c0;
    float xv[BLK], yv[BLK], bv[BLK];
#pragma unroll
    for (int s = 0; s < BLK; ++s) {
        const int k = kb + 4 * s + lg;
        bv[s] = b(k, n0 + li);
        xv[s] = a1(m0 + li, k);
        yv[s] = a2(m0 + li, k);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int blk = 0; blk < KSTEPS; blk += BLK) {
        float xn[BLK], yn[BLK], bn[BLK];
        if (blk + BLK < KSTEPS) {
#pragma unroll
            for (int s = 0; s < BLK; ++s) {
                const int k = kb + 4 * (blk + BLK + s) + lg;
                bn[s] = b(k, n0 + li);
                xn[s] = a1(m0 + li, k);
                yn[s] = a2(m0 + li, k);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < BLK; s += 2) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[s], bv[s], c0, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(yv[s], bv[s], d0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[s + 1], bv[s + 1], c1, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(yv[s + 1], bv[s + 1], d1, 0, 0, 0);
        }
        if (blk + BLK < KSTEPS) {
#pragma unroll
            for (int s = 0; s < BLK; ++s) {
                xv[s] = xn[s];
                yv[s] = yn[s];
                bv[s] = bn[s];
            }
        }
    }
    r1 = c0 + c1;
    r2 = d0 + d1;
}

// The same over k < m0 + 16: a product with a lower-triangular left operand
// (zero for k > m), so output rows m0 .. m0 + 15 need only the first m0 + 16 k.
template <int CC, class FA, class FB>
__device__ __forceinline__ f32x4 mfma_tile_lower(FA a, FB b, int m0, int n0)
{
    switch (m0 >> 4) {
    case 0:
        return mfma_tile<4>(a, b, m0, n0);
    case 1:
        return mfma_tile<8>(a, b, m0, n0);
    case 2:
        if constexpr (CC > 32)
            return mfma_tile<12>(a, b, m0, n0);
        break;
    default:
        if constexpr (CC > 32)
            return mfma_tile<16>(a, b, m0, n0);
        break;
    }
    return f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------- workspace

struct GenWs {
    size_t chunk_seq, chunk_start, chunk_len, seq_chunk0, seq_order, q, ke, w, u, aq, dec, onorm, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// MC = the chunk count bound (total / chunk + N); per (chunk, k-head) the
// normalised q rows, per (chunk, v-head) (diag(e) K)^T, W and scale * Aqk, each
// as a [hi block][lo block] pair of bf16 arrays (4 bytes a value), and U and
// three decay rows in f32; with the gated norm an f32 core output.
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
    L.seq_order = take(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    L.q = take(sizeof(float) * MC * Hk * C * dk);
    L.ke = take(sizeof(float) * MC * Hv * C * dk);
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
    // The carry takes sequences longest first: its workgroups are sequential
    // chains as long as their sequence, so the long ones start first and the
    // short ones fill in behind. Up to 1024 sequences are ranked by length (ties
    // by index); more keep their order.
    for (int i = threadIdx.x; i < p.N; i += 256) {
        int rank = i;
        if (p.N <= 1024) {
            const int li = p.cu[i + 1] - p.cu[i];
            rank = 0;
            for (int j = 0; j < p.N; ++j) {
                const int lj = p.cu[j + 1] - p.cu[j];
                rank += lj > li || (lj == li && j < i);
            }
        }
        p.seq_order[rank] = i;
    }
}

// ---------------------------------------------------------------- 2. prep

constexpr int kPrepThreads = 512;  // 8 waves

template <int DK, int DV>
__global__ __launch_bounds__(kPrepThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void prep_generic_kernel(
    PrefillParams p)
{
    constexpr int CC = gen_chunk<DK>();
    constexpr int NT = kPrepThreads, NW = NT / 64, NB = CC / 16;
    // v columns staged in LDS per pass
    constexpr int VSL = (CC == 64 && DK >= 128) ? 64 : (DV < 128 ? DV : 128);
    // pitches: PA, PC for rows read by m or n index, PB, PV by the contracted index
    constexpr int PA = DK + 2, PB = DK + 16, PC = CC + 2, PV = VSL + 16;
    constexpr int PQB = PA > PB ? PA : PB;
    static_assert(DV % VSL == 0 && CC % 16 == 0 && DK % 16 == 0 && CC * CC % NT == 0 && CC * DK % NT == 0 &&
                      CC * VSL % NT == 0 && CC % NW == 0 && NB - 1 <= NW,
                  "shape");

    __shared__ float Kc[CC][PA];     // the chunk's normalised keys
    __shared__ float QKb[CC * PQB];  // its normalised queries [CC][PA], then diag(beta gamma) K [CC][PB]
    __shared__ float Am[CC][PC];     // A (strictly lower), per v-head
    __shared__ float Tm[CC][PC];     // T = (I + A)^-1
    __shared__ float Vb[CC][PV];     // diag(beta) V, VSL columns
    __shared__ float G_s[CC], beta_s[CC], bg_s[CC], e_s[CC];
    auto Qc = [&](int r, int c) -> float & { return QKb[r * PA + c]; };
    auto Kb = [&](int r, int c) -> float & { return QKb[r * PB + c]; };

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv, Hk = hc.Hk, G = Hv / Hk;
    const int chunk = blockIdx.x / Hk, kh = blockIdx.x % Hk;
    const bool one_seq = p.N == 1;  // tokens [0, total): no table
    const int64_t tok0 = one_seq ? (int64_t)CC * chunk : p.chunk_start[chunk];
    const int n = one_seq ? min(CC, p.total - CC * chunk) : p.chunk_len[chunk];
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
    const uint32_t flags = hc.flags;
    const bool raw = flags & F_RAW_GATES;
    const int qdt = in.qkv_dt;
    auto vhead = [&](int j) { return hc.head_map == 0 ? kh * G + j : kh + j * Hk; };
    const void *gsa = raw ? in.a : static_cast<const void *>(in.g);
    const void *gsb = raw ? in.b : static_cast<const void *>(in.beta);
    const int gdt = raw ? in.ab_dt : DT_F32;

    // the gate words of one v-head (wave 0, lane = token), loaded a v-head ahead
    GateWord ga{0u}, gb{0u};
    auto load_gates = [&](int j) {
        const int64_t gi = (tok0 + min(lane, n - 1)) * Hv + vhead(j);
        ga = load_gate(gsa, gi, gdt);
        gb = load_gate(gsb, gi, gdt);
    };
    if (wave == 0)
        load_gates(0);

    // -- keys and queries: every load issued before any use, no branch around a
    // load (rows past the chunk's end re-read row n-1, columns past dk re-read
    // column dk-1, both masked after; the 32-bit word holding each element -- a
    // q/k row has an even length from a 4-element aligned start, so the word stays
    // in the row -- and the dtype by a select). Wave w takes rows w, w + 8, ...;
    // lane l columns l, l + 64, ...
    {
        constexpr int RW = CC / NW, EPL = (DK + 63) / 64;
        uint32_t kw[RW][EPL], qw[RW][EPL];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int64_t row = tok0 + min(wave + NW * i, n - 1);
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int c = min(lane + 64 * m, DK - 1);
                kw[i][m] = load_word_nb(in.k, row * in.k_stride + (int64_t)kh * DK + c, qdt);
                qw[i][m] = load_word_nb(in.q, row * in.q_stride + (int64_t)kh * DK + c, qdt);
            }
        }
        float *gq = p.gq + ((int64_t)chunk * Hk + kh) * CC * DK;
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int r = wave + NW * i;
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
                    Qc(r, c) = qv[m] * iq;
                    put_pair(gq, CC * DK, r * DK + c, qv[m] * iq);
                }
            }
        }
    }
    __syncthreads();

    // -- K K^T and Q K^T on the 16 x 16 tiles on and below the diagonal (A and
    // Aqk are lower triangular), one read of the keys for both; each wave keeps its
    // tiles (u = wave, wave + NW, ...) in registers for every v-head
    constexpr int NTRI = NB * (NB + 1) / 2, NTW = (NTRI + NW - 1) / NW;
    f32x4 gk[NTW], gq2[NTW];
    int tmw[NTW], tnw[NTW];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        const int u = wave + NW * k;
        int tm = 0, tn = u;  // u = tm (tm + 1) / 2 + tn, tn <= tm
        while (tn > tm) {
            tn -= tm + 1;
            ++tm;
        }
        tmw[k] = tm;
        tnw[k] = tn;
        if (u < NTRI)
            mfma_tile2<DK / 4>([&](int t, int i) { return Kc[t][i]; }, [&](int t, int i) { return Qc(t, i); },
                               [&](int i, int s2) { return Kc[s2][i]; }, 16 * tm, 16 * tn, 0, gk[k], gq2[k]);
    }

    constexpr int VPT = CC * VSL / NT;
    uint32_t vw[VPT];
    for (int j = 0; j < G; ++j) {
        const int h = vhead(j);
        // this v-head's first VSL columns of v, in flight from here
        auto load_v = [&](int d0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + NT * i;
                const int64_t row = tok0 + min(e / VSL, n - 1);
                vw[i] = load_word_nb(in.v, row * in.v_stride + (int64_t)h * DV + d0 + e % VSL, qdt);
            }
        };
        load_v(0);
        __syncthreads();  // the products are in LDS; the previous v-head is done with its buffers
        // -- gates and their in-chunk prefix sums (wave 0, lane = token); tokens
        // past the chunk's end get g = beta = 0, so they carry G_{n-1}
        float *dec = p.gdec + ((int64_t)chunk * Hv + h) * 3 * CC;
        if (wave == 0) {
            float g = gate_value(ga, gdt), beta = gate_value(gb, gdt);
            if (j + 1 < G)
                load_gates(j + 1);
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
                const float gam = expf(Gc), ed = expf(Glast - Gc);
                G_s[lane] = Gc;
                beta_s[lane] = beta;
                bg_s[lane] = beta * gam;
                e_s[lane] = ed;
                dec[lane] = hc.scale * gam;  // the output's decay (scale folded in)
                dec[CC + lane] = ed;         // the state update's decay
                dec[2 * CC + lane] = gam;    // gamma_t (gamma_last at CC - 1)
            }
        }
        __syncthreads();
        // -- A and scale * Aqk (to the workspace); diag(beta gamma) K for W and
        // diag(e) K (to the workspace) for the state update. Only the tiles on and
        // below the diagonal of K K^T and Q K^T were computed: select, not scale.
        {
            float *aq = p.gaq + ((int64_t)chunk * Hv + h) * CC * CC;
            // the tiles this wave holds: lane (li, lg) has rows 16 tm + 4 lg + r,
            // column 16 tn + li
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
                if (wave + NW * k < NTRI) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * tmw[k] + 4 * lg + r, s2 = 16 * tnw[k] + li;
                        const float dg = s2 <= t ? expf(G_s[t] - G_s[s2]) : 0.f;
                        Am[t][s2] = s2 < t ? beta_s[t] * dg * gk[k][r] : 0.f;
                        put_pair(aq, CC * CC, t * CC + s2, s2 <= t ? hc.scale * dg * gq2[k][r] : 0.f);
                    }
                }
            }
            // zeros above the diagonal tiles (A's are never read; Aqk's are)
#pragma unroll
            for (int i = 0; i < CC * CC / NT; ++i) {
                const int e = tid + NT * i, t = e / CC, s2 = e % CC;
                if (s2 / 16 > t / 16)
                    put_pair(aq, CC * CC, e, 0.f);
            }
            float *ke = p.gke + ((int64_t)chunk * Hv + h) * CC * DK;
#pragma unroll
            for (int i = 0; i < CC * DK / NT; ++i) {
                const int e = tid + NT * i, t = e / DK, c = e % DK;
                Kb(t, c) = bg_s[t] * Kc[t][c];
            }
            // (diag(e) K)^T, [dk][token]: consecutive threads take consecutive tokens
#pragma unroll
            for (int i = 0; i < CC * DK / NT; ++i) {
                const int e = tid + NT * i, c = e / CC, t = e % CC;
                put_pair(ke, CC * DK, e, e_s[t] * Kc[t][c]);
            }
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
        // (b) the blocks below the diagonal, one sub-diagonal after another, a wave
        // per block: T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj). The inner sum M
        // stays in the accumulator; the product with T_ii then pairs k-step kk and
        // row-of-four lg with contraction index 4 lg + kk, the row of M that the
        // lane holds in element kk.
        for (int L = 1; L < NB; ++L) {
            if (wave < NB - L) {
                const int jb = wave, ib = wave + L;
                f32x4 m = {0.f, 0.f, 0.f, 0.f};
                for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int k = 16 * kb + 4 * kk + lg;
                        m = __builtin_amdgcn_mfma_f32_16x16x4f32(Am[16 * ib + li][k], Tm[k][16 * jb + li], m, 0, 0,
                                                                 0);
                    }
                }
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[16 * ib + li][16 * ib + 4 * lg + kk], m[kk], t, 0,
                                                             0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Tm[16 * ib + 4 * lg + r][16 * jb + li] = -t[r];
            }
            __syncthreads();
        }
        // -- W = T diag(beta gamma) K and U = T diag(beta) V (to the workspace), v
        // staged VSL columns at a time; T is lower triangular, so each output row
        // block contracts over the chunk's first m0 + 16 tokens only (longest first)
        float *wg = p.gw + ((int64_t)chunk * Hv + h) * CC * DK;
        float *ug = p.gu + ((int64_t)chunk * Hv + h) * CC * DV;
        constexpr int NWT = NB * (DK / 16), NUT = NB * (VSL / 16);
        for (int d0 = 0; d0 < DV; d0 += VSL) {
            if (d0 > 0) {
                load_v(d0);
                __syncthreads();  // the previous pass is done with Vb
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + NT * i, r = e / VSL, jj = e % VSL;
                Vb[r][jj] = r < n ? beta_s[r] * word_to_f32(vw[i], jj, qdt) : 0.f;
            }
            __syncthreads();
            const int first = d0 == 0 ? 0 : NWT;
            for (int u = first + wave; u < NWT + NUT; u += NW) {
                if (u < NWT) {
                    const int m0 = (NB - 1 - u / (DK / 16)) * 16, n0 = (u % (DK / 16)) * 16;
                    const f32x4 acc = mfma_tile_lower<CC>([&](int t, int s2) { return Tm[t][s2]; },
                                                          [&](int s2, int i) { return Kb(s2, i); }, m0, n0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        put_pair(wg, CC * DK, (m0 + 4 * lg + r) * DK + n0 + li, acc[r]);
                } else {
                    const int v = u - NWT;
                    const int m0 = (NB - 1 - v / (VSL / 16)) * 16, n0 = (v % (VSL / 16)) * 16;
                    const f32x4 acc = mfma_tile_lower<CC>([&](int t, int s2) { return Tm[t][s2]; },
                                                          [&](int s2, int jj) { return Vb[s2][jj]; }, m0, n0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ug[(m0 + 4 * lg + r) * DV + d0 + n0 + li] = acc[r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- 3. carry

constexpr int kCarryThreads = 512;  // 8 waves, two per SIMD

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 of an LDS row
__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// C[m][n] += sum_k A[m][k] B[n][k] over k in [0, 32 KB) for a 16 x 16 tile, both
// operands bf16 hi/lo pairs in LDS rows with k contiguous (pitches PA, PB). Lane
// (li, lg) feeds A[m0 + li][32 kb + 8 lg ..] and B[n0 + li][32 kb + 8 lg ..] and
// receives C[m0 + 4 lg + r][n0 + li] in element r; hi*hi in one chain, hi*lo +
// lo*hi in another.
template <int KB, int PA, int PB>
__device__ __forceinline__ f32x4 tile_pair(const uint16_t *ah, const uint16_t *al, const uint16_t *bh,
                                           const uint16_t *bl, int m0, int n0, f32x4 c)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int ao = (m0 + li) * PA + 8 * lg, bo = (n0 + li) * PB + 8 * lg;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a1 = lds8(ah + ao + 32 * kb), a2 = lds8(al + ao + 32 * kb);
        const bf16x8 b1 = lds8(bh + bo + 32 * kb), b2 = lds8(bl + bo + 32 * kb);
        c = mfma_bf16(a1, b1, c);
        x = mfma_bf16(a1, b2, x);
        x = mfma_bf16(a2, b1, x);
    }
    return c + x;
}

// Two tiles that share B: A1 B and A2 B (one read of B for both).
template <int KB, int PA, int PB>
__device__ __forceinline__ void tile_pair2(const uint16_t *a1h, const uint16_t *a1l, const uint16_t *a2h,
                                           const uint16_t *a2l, const uint16_t *bh, const uint16_t *bl, int m0,
                                           int n0, f32x4 &r1, f32x4 &r2)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int ao = (m0 + li) * PA + 8 * lg, bo = (n0 + li) * PB + 8 * lg;
    f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, x1 = c1, c2 = c1, x2 = c1;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 b1 = lds8(bh + bo + 32 * kb), b2 = lds8(bl + bo + 32 * kb);
        const bf16x8 p1 = lds8(a1h + ao + 32 * kb), p2 = lds8(a1l + ao + 32 * kb);
        const bf16x8 q1 = lds8(a2h + ao + 32 * kb), q2 = lds8(a2l + ao + 32 * kb);
        c1 = mfma_bf16(p1, b1, c1);
        c2 = mfma_bf16(q1, b1, c2);
        x1 = mfma_bf16(p1, b2, x1);
        x2 = mfma_bf16(q1, b2, x2);
        x1 = mfma_bf16(p2, b1, x1);
        x2 = mfma_bf16(q2, b1, x2);
    }
    r1 = c1 + x1;
    r2 = c2 + x2;
}

// Per (sequence, v-head, 32 dv rows). The slice's state is held in f32 MFMA
// accumulators for the whole call: each wave owns fixed 16 x 16 state tiles
// (rows dv, columns dk), updates them in place every chunk and publishes them to
// LDS as bf16 hi/lo for the next chunk's Q S^T and W S^T. Every product is three
// bf16 MFMAs (hi*hi + hi*lo + lo*hi) on operands the preparation kernel stored as
// hi/lo pairs.
template <int DK, int DV>
__global__ __launch_bounds__(kCarryThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void carry_generic_kernel(
    PrefillParams p)
{
    constexpr int CC = gen_chunk<DK>();
    constexpr int NT = kCarryThreads, NW = NT / 64;
    constexpr int NSL = DV / kSlice;
    // bf16 row pitches: rows 16-byte aligned, and 8 consecutive rows start in 8
    // different 16-byte bank groups (the 16-byte operand reads take 8 lanes a pass)
    constexpr int PK = DK + 8, PC = CC + 8;
    constexpr int NT1 = (CC / 16) * (kSlice / 16);  // Q S^T / W S^T tiles = output tiles
    constexpr int NU = (kSlice / 16) * (DK / 16);   // state tiles
    constexpr int NUW = (NU + NW - 1) / NW;         // state tiles per wave
    constexpr int KB = DK / 32, CB = CC / 32;       // 32-wide k blocks over dk, over the chunk
    // 16-byte pieces of one chunk's operands (hi and lo halves): q, W and
    // (diag(e) K)^T split evenly over the threads, Aqk may leave whole waves idle
    constexpr int NQ = 2 * CC * DK / 8, NA = 2 * CC * CC / 8;
    constexpr int WQ = NQ / NT, WA = (NA + NT - 1) / NT;
    static_assert(NT1 == NW || 2 * NT1 == NW, "phase-1 tiles");
    static_assert(NQ % NT == 0 && NA % 64 == 0 && DK % 32 == 0 && CC % 32 == 0 && 3 * CC <= NT, "shape");

    __shared__ __attribute__((aligned(16))) uint16_t Sh[kSlice][PK], Sl[kSlice][PK];  // S[j][i], hi / lo
    __shared__ __attribute__((aligned(16))) uint16_t Qh[CC][PK], Ql[CC][PK];          // normalised q rows
    __shared__ __attribute__((aligned(16))) uint16_t Wh[CC][PK], Wl[CC][PK];          // W rows
    __shared__ __attribute__((aligned(16))) uint16_t Kh[DK][PC], Kl[DK][PC];          // (diag(e) K)^T
    __shared__ __attribute__((aligned(16))) uint16_t Dh[kSlice][PC], Dl[kSlice][PC];  // D^T of the slice
    __shared__ __attribute__((aligned(16))) uint16_t Ah[CC][PC], Al[CC][PC];          // scale * Aqk
    __shared__ float Dc[3][CC];  // scale gamma_t, exp(G_last - G_t), gamma_t

    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv, Hk = hc.Hk;
    const int slice = blockIdx.x % NSL;
    const int h = (blockIdx.x / NSL) % Hv;
    const int kh = k_head_of(hc.head_map, h, Hk, Hv);
    const int seq = p.N == 1 ? 0 : p.seq_order[blockIdx.x / (NSL * Hv)];  // longest first
    const int dv0 = slice * kSlice;
    const bool one_seq = p.N == 1;
    const int start = one_seq ? 0 : p.cu[seq];
    const int len = one_seq ? p.total : p.cu[seq + 1] - start;
    if (len <= 0)
        return;  // empty sequence: state untouched
    const int nch = (len + CC - 1) / CC;
    const int cfirst = one_seq ? 0 : p.seq_chunk0[seq];
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
    const uint32_t flags = hc.flags;
    float *Sg = p.state + (((int64_t)seq * Hv + h) * DV + dv0) * DK;
    void *obase = (flags & F_GATED_NORM) ? static_cast<void *>(p.onorm) : p.out;
    const int odt = (flags & F_GATED_NORM) ? DT_F32 : p.out_dt;

    // phase-1 tile of this wave: rows m1 (tokens), columns n1 (dv). With a tile per
    // wave the wave forms Q S^T and D; with two waves per tile (32-token chunks)
    // the first forms Q S^T, the second D. The Q S^T wave also owns the output tile.
    const int t1 = NT1 == NW ? wave : wave % NT1;
    const int m1 = (t1 / (kSlice / 16)) * 16, n1 = (t1 % (kSlice / 16)) * 16;
    const bool makes_q = NT1 == NW || wave < NT1, makes_d = NT1 == NW || wave >= NT1;

    // the state tiles this wave owns: tile u = wave + NW k, rows (dv) 16 (u % 2),
    // columns (dk) 16 (u / 2)
    f32x4 S[NUW];
    auto publish = [&](int k, int u) {  // the tile's bf16 hi / lo for the next Q S^T, W S^T
        const int m0 = (u % 2) * 16, n0 = (u / 2) * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            bf16_split(S[k][r], Sh[m0 + 4 * lg + r][n0 + li], Sl[m0 + 4 * lg + r][n0 + li]);
    };
#pragma unroll
    for (int k = 0; k < NUW; ++k) {
        const int u = wave + NW * k;
        if (u < NU) {
            const int m0 = (u % 2) * 16, n0 = (u / 2) * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[k][r] = Sg[(m0 + 4 * lg + r) * DK + n0 + li];
            publish(k, u);
        }
    }

    // one chunk's operands in registers: 16-byte piece tid + NT i of each array;
    // U at this wave's phase-1 tile positions (the D wave only)
    uint4 rq[WQ], rw[WQ], rk[WQ], ra[WA];
    float ru[4] = {0.f, 0.f, 0.f, 0.f}, rd;
    auto fetch = [&](int ci) {
        const int64_t c = cfirst + ci;
        const uint4 *gq = reinterpret_cast<const uint4 *>(p.gq + (c * Hk + kh) * CC * DK);
        const uint4 *gk = reinterpret_cast<const uint4 *>(p.gke + (c * Hv + h) * CC * DK);
        const uint4 *gw = reinterpret_cast<const uint4 *>(p.gw + (c * Hv + h) * CC * DK);
        const uint4 *ga = reinterpret_cast<const uint4 *>(p.gaq + (c * Hv + h) * CC * CC);
#pragma unroll
        for (int i = 0; i < WQ; ++i) {
            rq[i] = gq[tid + NT * i];
            rw[i] = gw[tid + NT * i];
            rk[i] = gk[tid + NT * i];
        }
#pragma unroll
        for (int i = 0; i < WA; ++i) {
            const int e = tid + NT * i;
            if (e < NA)
                ra[i] = ga[e];
        }
        if (makes_d) {
            const float *gu = p.gu + (c * Hv + h) * CC * DV + dv0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ru[r] = gu[(m1 + 4 * lg + r) * DV + n1 + li];
        }
        rd = p.gdec[(c * Hv + h) * 3 * CC + min(tid, 3 * CC - 1)];
    };
    // piece e of a [hi block][lo block] pair of row-major arrays with `len` values a
    // row (nh pieces a block) into LDS rows of `pitch` bf16; the hi/lo choice is
    // uniform over a wave (nh is a multiple of 64)
    auto put8 = [](uint16_t *hi, uint16_t *lo, int pitch, int len, int nh, int e, uint4 v) {
        const bool second = e >= nh;
        const int e2 = second ? e - nh : e;
        *reinterpret_cast<uint4 *>((second ? lo : hi) + (8 * e2 / len) * pitch + (8 * e2) % len) = v;
    };
    fetch(0);

    for (int ci = 0; ci < nch; ++ci) {
        const int n = min(CC, len - ci * CC);
        const int64_t tok0 = start + (int64_t)ci * CC;
        __syncthreads();  // the previous chunk is done with every buffer; S published
#pragma unroll
        for (int i = 0; i < WQ; ++i) {
            const int e = tid + NT * i;
            put8(&Qh[0][0], &Ql[0][0], PK, DK, NQ / 2, e, rq[i]);
            put8(&Wh[0][0], &Wl[0][0], PK, DK, NQ / 2, e, rw[i]);
            put8(&Kh[0][0], &Kl[0][0], PC, CC, NQ / 2, e, rk[i]);
        }
#pragma unroll
        for (int i = 0; i < WA; ++i) {
            const int e = tid + NT * i;
            if (e < NA)
                put8(&Ah[0][0], &Al[0][0], PC, CC, NA / 2, e, ra[i]);
        }
        if (tid < 3 * CC)
            Dc[tid / CC][tid % CC] = rd;
        float uc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            uc[r] = ru[r];
        if (ci + 1 < nch)
            fetch(ci + 1);  // the next chunk's operands, in flight from here
        __syncthreads();

        // -- Q S^T and D = U - W S^T on the entering state; this wave keeps
        // scale gamma_t (Q S^T) of its output tile in registers and publishes D^T
        f32x4 qv = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NT1 == NW) {
            tile_pair2<KB, PK, PK>(&Qh[0][0], &Ql[0][0], &Wh[0][0], &Wl[0][0], &Sh[0][0], &Sl[0][0], m1, n1, qv, wv);
        } else if (makes_q) {
            qv = tile_pair<KB, PK, PK>(&Qh[0][0], &Ql[0][0], &Sh[0][0], &Sl[0][0], m1, n1, qv);
        } else {
            wv = tile_pair<KB, PK, PK>(&Wh[0][0], &Wl[0][0], &Sh[0][0], &Sl[0][0], m1, n1, wv);
        }
        if (makes_q) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                qv[r] *= Dc[0][m1 + 4 * lg + r];
        }
        if (makes_d) {  // D^T[j][t]: this lane's 4 consecutive tokens of row j
            uint16_t dh[4], dl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bf16_split(uc[r] - wv[r], dh[r], dl[r]);
            *reinterpret_cast<uint2 *>(&Dh[n1 + li][m1 + 4 * lg]) =
                make_uint2(dh[0] | ((uint32_t)dh[1] << 16), dh[2] | ((uint32_t)dh[3] << 16));
            *reinterpret_cast<uint2 *>(&Dl[n1 + li][m1 + 4 * lg]) =
                make_uint2(dl[0] | ((uint32_t)dl[1] << 16), dl[2] | ((uint32_t)dl[3] << 16));
        }
        __syncthreads();

        // -- the state update S <- gamma_last S + D^T (diag(e) K) on this wave's
        // tiles (contracting over the chunk's tokens), published for the next chunk
        const float gl = Dc[2][CC - 1];
#pragma unroll
        for (int k = 0; k < NUW; ++k) {
            const int u = wave + NW * k;
            if (u < NU) {
                S[k] = tile_pair<CB, PC, PC>(&Dh[0][0], &Dl[0][0], &Kh[0][0], &Kl[0][0], (u % 2) * 16,
                                             (u / 2) * 16, S[k] * gl);
                publish(k, u);
            }
        }
        // -- the output tile: O = scale gamma (Q S^T) + (scale Aqk) D, contracting
        // only over the 32-token blocks at or below the tile's last row (Aqk is
        // zero above the diagonal)
        if (makes_q) {
            f32x4 o = qv;
            if (m1 < 32)
                o = tile_pair<1, PC, PC>(&Ah[0][0], &Al[0][0], &Dh[0][0], &Dl[0][0], m1, n1, o);
            else
                o = tile_pair<CB, PC, PC>(&Ah[0][0], &Al[0][0], &Dh[0][0], &Dl[0][0], m1, n1, o);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m1 + 4 * lg + r;
                if (t < n)
                    store_act(obase, ((tok0 + t) * Hv + h) * DV + dv0 + n1 + li, odt, o[r]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NUW; ++k) {
        const int u = wave + NW * k;
        if (u < NU) {
            const int m0 = (u % 2) * 16, n0 = (u / 2) * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sg[(m0 + 4 * lg + r) * DK + n0 + li] = S[k][r];
        }
    }
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
                       dim3(kPrepThreads), 0, s, p);
    hipLaunchKernelGGL((carry_generic_kernel<DK, DV>), dim3((unsigned)((int64_t)p.N * p.hc.Hv * (DV / kSlice))),
                       dim3(kCarryThreads), 0, s, p);
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

int prefill_generic_carry_threads() { return kCarryThreads; }

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
    p.seq_order = reinterpret_cast<int32_t *>(b + L.seq_order);
    p.gq = reinterpret_cast<float *>(b + L.q);
    p.gke = reinterpret_cast<float *>(b + L.ke);
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
