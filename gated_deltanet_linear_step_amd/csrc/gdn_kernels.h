// gdn_kernels.h -- kernel parameter blocks and launchers (host side of the kernels).
// The C ABI layer (gdn_api.cpp) validates arguments, fills these blocks and
// calls the launchers; each launcher returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ActInputs {
    const void *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    int qkv_dt;
    const void *a, *b;
    int ab_dt;
    const float *decay_param, *dt_bias;
    const float *g, *beta;
    const void *z;
    int z_dt;
    const float *norm_w;
};

struct HeadCfg {
    int Hk, Hv, dk, dv, head_map, decay_kind;
    uint32_t flags;
    float scale, l2_eps, norm_eps;
};

struct DecodeParams {
    ActInputs in;
    HeadCfg hc;
    float *state;
    const int32_t *slots;
    int num_slots;
    void *out;
    int out_dt;
    int B, T;
    // gdn_decode_layer: q/k/v are pre-conv; conv_k > 0 applies the causal conv
    // (weights [channels][K], state [slots][channels][K-1], ping-pong in/out)
    int conv_k;
    const void *conv_w, *conv_in;
    void *conv_out;
};

struct ConvParams {
    int C, K, N, total, uniform_len;
    const int32_t *cu;
    const void *x;
    int64_t x_stride;
    const void *w;
    void *state;
    void *y;
    int64_t y_stride;
    int x_dt, y_dt;
};

// Prefill geometry: 64-token chunks that start at each sequence's first token.
constexpr int kChunk = 64;

struct PrefillParams {
    ActInputs in;
    HeadCfg hc;
    float *state;
    void *out;
    int out_dt;
    int N, total;
    const int32_t *cu;  // device [N+1]
    int num_chunks;     // sum over sequences of ceil(len / chunk length)
    int max_seq_chunks; // largest per-sequence chunk count
    // workspace carve-out (device pointers)
    int32_t *chunk_seq;    // [num_chunks] sequence of each chunk
    int32_t *chunk_start;  // [num_chunks] first packed token row
    int32_t *chunk_len;    // [num_chunks] tokens in the chunk (1..64)
    int32_t *seq_chunk0;   // [N] index of each sequence's first chunk
    int32_t *seq_order;    // [N] sequences longest first (the carry's order)
    uint16_t *qn;          // [num_chunks][Hk][64][dk]   f16, normalised q rows
    uint16_t *knT;         // [num_chunks][Hk][dk][64]   f16, normalised k, transposed
    uint16_t *wmat;        // [num_chunks][Hv][64][dk]   f16, W = T diag(beta*gamma) K
    float *umat;           // [num_chunks][Hv][dv][64]   f32, -U^T with U = T diag(beta) V
    uint16_t *aqk;         // [num_chunks][Hv][64][64]   f16, -scale (masked decayed Q K^T)
    float *gcum;           // [num_chunks][Hv][4][64]    f32, exp(G_t), -exp(G_last - G_t), scale exp(G_t), 0
    float *onorm;          // [total][Hv][dv]            f32 core output (gated norm only)
    // the f32-accuracy path of the other head shapes (C = its chunk length): gq,
    // gke, gw and gaq hold per (chunk, head) a bf16 hi block then a bf16 lo block
    // (4 bytes a value); gu and gdec are f32
    float *gq;             // [num_chunks][Hk][C][dk]    normalised q rows
    float *gke;            // [num_chunks][Hv][dk][C]    (diag(exp(G_last - G_t)) K)^T (normalised k)
    float *gw;             // [num_chunks][Hv][C][dk]    W = T diag(beta gamma) K
    float *gu;             // [num_chunks][Hv][C][dv]    U = T diag(beta) V
    float *gaq;            // [num_chunks][Hv][C][C]     scale * (masked decayed Q K^T)
    float *gdec;           // [num_chunks][Hv][3][C]     scale gamma_t, exp(G_last - G_t), gamma_t
};

// Which decode kernel a call runs: waves per workgroup, lanes per state row, token
// mode (0 any count, 1 fused-layer token groups, 2 one token), non-temporal state
// access, workgroups and threads per workgroup. launch_decode launches exactly this.
struct DecodePlan {
    int waves, lanes_per_row, mode, nontemporal, workgroups, threads;
};
bool decode_supported(int dk, int dv);
DecodePlan decode_plan(int dk, int dv, int B, int T, int Hv, bool fused_conv, uint32_t flags);
hipError_t launch_decode(const DecodeParams &p, hipStream_t s);
hipError_t launch_conv(const ConvParams &p, hipStream_t s);
// Which carry kernel a prefill runs: kind 0 = carry_split (compute and output waves
// per slice), 1 = carry (one wave per slice), 2 = the carry of the f32-accuracy
// path of the other head shapes (32 dv rows per workgroup); dv slices of 16 rows per workgroup;
// carry workgroups and threads per workgroup; prep workgroups. launch_prefill
// launches exactly this for the device's compute-unit count.
struct PrefillPlan {
    int carry_kind, slices_per_wg, carry_workgroups, carry_threads, prep_workgroups;
};
bool prefill_supported(int dk, int dv);
// The f32-accuracy path (gdn_prefill_generic.hip) for the shapes other than 128 x 128.
bool prefill_generic_supported(int dk, int dv);
int prefill_generic_chunk(int dk);
int prefill_generic_carry_threads();  // threads per carry workgroup of the f32 path
size_t prefill_generic_workspace_bytes(int Hk, int Hv, int dk, int dv, int64_t max_chunks, int N,
                                       int64_t total_tokens, bool norm);
void prefill_generic_carve(PrefillParams &p, void *ws, int64_t max_chunks);
hipError_t launch_prefill_generic(const PrefillParams &p, hipStream_t s);
// Tokens per chunk of the prefill that serves (dk, dv): 64, or 32 for the f32 path at dk = 256.
int prefill_chunk_len(int dk, int dv);
PrefillPlan prefill_plan(int N, int Hk, int Hv, int dk, int dv, int64_t num_chunks, int cus);
size_t prefill_workspace_bytes(int Hk, int Hv, int dk, int dv, int64_t max_chunks, int N,
                               int64_t total_tokens, bool norm);
void prefill_carve(PrefillParams &p, void *ws, int64_t max_chunks);
hipError_t launch_prefill(const PrefillParams &p, hipStream_t s);

}  // namespace gdn
