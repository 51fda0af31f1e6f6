/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta-rule library, libgdn.so.
 *
 * The library computes one gated delta-rule linear-attention layer core: the
 * per-token, per-value-head recurrence on an fp32 state S[dv][dk]
 *
 *     S <- exp(g) * S;   p = S k;   d = beta * (v - p);   S <- S + d k^T;   o = (S q) / sqrt(dk)
 *
 * (module doc of docs.rs ferrox-core 0.24.0 src/gdn.rs, `delta_step`; CPU reference
 * `cpu_segment` of docs.rs ferrum-kernels 0.8.0
 * src/backend/metal/vnext_ops/gated_delta_attention_tests.rs), plus the ops that
 * surround it in that reference: depthwise causal conv + SiLU with carried raw
 * inputs, L2 norm of q and k, the softplus/sigmoid gates, the grouped or tiled
 * k-head map, and the gated RMS norm of the output.
 *
 * Conventions shared by every entry point
 *  - Every array pointer is a DEVICE pointer unless its comment says "host".
 *    The caller owns all memory; the library allocates nothing and keeps no
 *    state between calls.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream). Results are visible after the stream is synchronised. Calls are
 *    reentrant; calls that share output or state buffers must be ordered by the
 *    caller (same stream or events).
 *  - All arguments are validated on the host before any HIP call. A call that
 *    returns an error status has launched nothing and changed no buffer.
 *    GDN_ERR_LAUNCH is the only status reported after a launch was attempted.
 *  - Nothing aborts, prints or throws across this interface.
 *  - dtypes: activations may be f32, f16 or bf16 (gdn_dtype); states, gates given
 *    as g/beta, decay parameters, dt_bias and norm weights are f32.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a pointer the configuration needs is NULL */
    GDN_ERR_SHAPE = 2,       /* inconsistent sizes: counts < 0, Hv % Hk != 0, bad cu_seqlens */
    GDN_ERR_UNSUPPORTED = 3, /* valid but not built: head dims, conv width, dtype, flags */
    GDN_ERR_OVERFLOW = 4,    /* an element count or offset exceeds what the kernels index */
    GDN_ERR_ALIGN = 5,       /* a pointer or stride breaks the alignment a kernel needs */
    GDN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size query returned */
    GDN_ERR_LAUNCH = 7,      /* the HIP runtime reported an error for a launch */
    GDN_ERR_SCRATCH = 8      /* gdn_prefill_chunked_noalloc: the call needs more workspace
                                than its static scratch (GDN_NOALLOC_SCRATCH_BYTES) */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2 } gdn_dtype;

/* Which k-head v-head h reads (docs.rs ferrox-core src/gdn.rs `HeadMap`;
 * ferrum-kernels tests page `GatedDeltaValueHeadMapping`):
 *   GROUPED: h / (Hv / Hk)   (Qwen3-Next order)
 *   TILED:   h % Hk          (Qwen3.5 order; "interleaved by key head")          */
typedef enum gdn_head_map { GDN_MAP_GROUPED = 0, GDN_MAP_TILED = 1 } gdn_head_map;

/* How the per-head decay parameter becomes the rate that multiplies softplus
 * (ferrum-kernels tests page, `cpu_segment` gate section):
 *   LOG_RATE:      rate = -exp(decay_param[h])   (decay_param is A_log)
 *   NEGATIVE_RATE: rate = decay_param[h]         (decay_param is -exp(A_log))   */
typedef enum gdn_decay { GDN_DECAY_LOG_RATE = 0, GDN_DECAY_NEGATIVE_RATE = 1 } gdn_decay;

/* gdn_dims.flags */
enum {
    /* q, k rows are normalised in-op: x * (sum x^2 + l2_eps)^(-1/2) per (token,
     * k-head) (ferrum-kernels tests page, `normalize_rows` and `cpu_segment`). */
    GDN_L2NORM_QK = 1u,
    /* gates from raw a, b: g = rate * softplus(a + dt_bias), beta = sigmoid(b)
     * (softplus with the +-20 cut-overs of that page's `softplus`). Without this
     * flag the caller passes g and beta directly. */
    GDN_RAW_GATES = 2u,
    /* output y = o * (mean_j o_j^2 + norm_eps)^(-1/2) * norm_weight * silu(z)
     * over the dv values of each (token, v-head) (that page's `cpu_segment`
     * output section). Without it the output is the core o itself. */
    GDN_GATED_NORM = 4u,
    /* Decode entry points only (the prefill returns UNSUPPORTED): a cache hint
     * for callers whose states do not stay in the GPU's last-level cache from
     * one call to the next (many layers or sequences, more state than the
     * cache holds). The state is loaded and stored with non-temporal hints;
     * results are bit for bit those of a call without the flag. On states the
     * cache does keep, the flag makes the step slower. */
    GDN_STREAM_STATE = 8u
};

typedef struct gdn_dims {
    int32_t num_k_heads; /* Hk >= 1 */
    int32_t num_v_heads; /* Hv >= 1, Hv % Hk == 0 */
    int32_t head_dim_k;  /* dk */
    int32_t head_dim_v;  /* dv. Built (dk, dv), for every entry point: (32,32), (64,64),
                            (96,96), (128,128), (64,128), (128,64), (128,256),
                            (256,128), (256,256). Others: UNSUPPORTED. */
    int32_t head_map;    /* gdn_head_map */
    int32_t decay;       /* gdn_decay, used with GDN_RAW_GATES */
    uint32_t flags;      /* GDN_L2NORM_QK | GDN_RAW_GATES | GDN_GATED_NORM |
                            GDN_STREAM_STATE */
    float scale;         /* read-out scale; 0 selects 1/sqrt(dk) */
    float l2_eps;        /* 0 selects 1e-6 */
    float norm_eps;      /* 0 selects 1e-6 */
} gdn_dims;

/* Per-token activations. A "token row" r indexes tokens: r = b * T + t for the
 * decode step (sequence b, token t of T) and the packed token index for the
 * prefill. Element (row r, head, i) of q is at q[r * q_stride + head * dk + i]
 * (same for k with k_stride, v with v_stride and dv), so q, k, v may be strided
 * views into one mixed [tokens][2*Hk*dk + Hv*dv] row. Strides are in elements.
 * The kernels read q, k and v in groups of 4 elements: each base pointer must be
 * aligned to 4 elements and each stride a multiple of 4 (else GDN_ERR_ALIGN). */
typedef struct gdn_inputs {
    const void *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    int32_t qkv_dtype;      /* gdn_dtype of q, k, v */
    /* GDN_RAW_GATES: a, b [tokens][Hv] contiguous in ab_dtype, aligned to their
     * element size; decay_param and dt_bias [Hv] f32. Every read stays within
     * the tokens*Hv elements. */
    const void *a, *b;
    int32_t ab_dtype;
    const float *decay_param, *dt_bias;
    /* no GDN_RAW_GATES: g (log decay, <= 0 in a real layer) and beta [tokens][Hv] f32,
     * 4-byte aligned */
    const float *g, *beta;
    /* GDN_GATED_NORM: z [tokens][Hv][dv] contiguous in z_dtype, 4-byte aligned
     * (read as 32-bit words; dv is even in every built shape, so no word reaches
     * past the last element); norm_weight [dv] f32 */
    const void *z;
    int32_t z_dtype;
    const float *norm_weight;
} gdn_inputs;

/* ---------------------------------------------------------------------------
 * gdn_conv_update -- depthwise causal conv1d + SiLU with carried raw inputs.
 * (ferrum-kernels tests page, `cpu_segment` conv section; docs.rs libmir-metal
 * 0.1.0 src/engine/gated_delta_layer/decode/mod.rs, `convolve`.)
 *
 * For sequence i with tokens [cu[i], cu[i+1]) and each channel c:
 *   y[r][c] = silu( sum_{m<K} weight[c][m] * xhat(t + m - (K-1)) ),  t = r - cu[i]
 * where xhat(j) = x[cu[i] + j][c] for j >= 0 and conv_state[i][c][(K-1) + j]
 * otherwise; afterwards conv_state[i][c][:] holds the last K-1 entries of
 * [old state || this call's inputs], oldest first. No bias. A zero-length
 * sequence leaves its state untouched.
 *
 *   channels      C >= 1
 *   kernel_size   K, 2 <= K <= 8
 *   num_seqs      N >= 0
 *   cu_seqlens    device int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = total_tokens;
 *                 NULL means every sequence has total_tokens / N tokens (N must divide it)
 *   x             [total_tokens] rows of x_stride elements (>= C), x_dtype
 *   weight        [C][K] in x_dtype
 *   conv_state    [N][C][K-1] in x_dtype, updated in place
 *   y             [total_tokens] rows of y_stride elements (>= C), y_dtype; may not alias x
 * Errors: NULL, SHAPE (counts, strides), UNSUPPORTED (K, dtype), OVERFLOW.
 * ------------------------------------------------------------------------- */
gdn_status gdn_conv_update(int32_t channels, int32_t kernel_size, int32_t num_seqs,
                           const int32_t *cu_seqlens, int32_t total_tokens, int32_t x_dtype,
                           const void *x, int64_t x_stride, const void *weight, void *conv_state,
                           int32_t y_dtype, void *y, int64_t y_stride, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_decode_step -- the recurrence for `batch` independent sequences of
 * `tokens_per_seq` tokens each, token order preserved, each sequence's state
 * read from HBM once and written once per call (ferrox-core src/gdn.rs
 * `delta_step` for one token; ferrum-kernels tests page `cpu_segment` for the
 * token loop, the gates and the gated norm).
 *
 *   dims            see gdn_dims; flags select L2 norm, raw gates, gated norm
 *   batch           B >= 0 sequences
 *   tokens_per_seq  T >= 1; token row of (b, t) is b*T + t
 *   in              activations; see gdn_inputs
 *   state           [num_slots][Hv][dv][dk] f32, key index innermost, 16-byte
 *                   aligned; updated in place
 *   state_slots     device int32 [B]: slot of sequence b; NULL means slot b.
 *                   A slot outside [0, num_slots) leaves that sequence's state
 *                   and output rows untouched.
 *   num_slots       number of state slots (>= B when state_slots is NULL)
 *   out_dtype, out  [B*T][Hv][dv]; may not alias any input or the state
 * Errors: NULL, SHAPE, UNSUPPORTED (dims, dtype), OVERFLOW, ALIGN (q/k/v groups of 4
 * elements; a, b to their element size; g, beta, z and norm_weight to 4 bytes; the
 * state to 16 bytes), LAUNCH.
 * ------------------------------------------------------------------------- */
gdn_status gdn_decode_step(const gdn_dims *dims, int32_t batch, int32_t tokens_per_seq,
                           const gdn_inputs *in, float *state, const int32_t *state_slots,
                           int32_t num_slots, int32_t out_dtype, void *out, void *stream);

/* The causal conv that gdn_decode_layer applies to q, k and v before the
 * recurrence: the same operation as gdn_conv_update over the channel order
 * [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)] of the mixed projection row. */
typedef struct gdn_conv_args {
    int32_t kernel_size;  /* K; the built layer kernel supports K = 4 */
    const void *weight;   /* [channels][K] in the activations' dtype (qkv_dtype) */
    const void *state_in; /* [num_slots][channels][K-1], oldest first, qkv_dtype */
    void *state_out;      /* same shape; must not overlap state_in */
} gdn_conv_args;

/* ---------------------------------------------------------------------------
 * gdn_decode_layer -- one launch for the whole decode layer: causal conv + SiLU
 * of q, k, v with carried raw inputs (ferrum-kernels tests page, `cpu_segment`
 * conv section; libmir-metal decode/mod.rs `convolve`), then everything
 * gdn_decode_step does (L2 norm, gates, recurrence, gated norm).
 *
 * Arguments are those of gdn_decode_step, except:
 *   in->q, in->k, in->v  the PRE-conv projections (e.g. views into the mixed
 *                        [tokens][2*Hk*dk + Hv*dv] row)
 *   conv                 weights and conv state; the state is indexed by the
 *                        same slot as the delta state. The call reads state_in
 *                        and writes the window after its tokens to state_out
 *                        (a caller alternates two buffers); both must be aligned
 *                        to 4 elements. A slot outside [0, num_slots) leaves both
 *                        states and the output rows untouched.
 * Every v-head workgroup computes the conv of the q/k channels it reads; the
 * new q/k window is written by one workgroup per k-head, which is why the
 * state is not updated in place.
 * Slot pools: a call writes new windows only for the slots it names (and a
 * live slot's window only to state_out); for every other slot state_out keeps
 * what it held. A caller that alternates the two buffers while some calls do
 * not name every slot must therefore carry the windows of the slots a call left
 * out: e.g. copy those slots' windows from state_in to state_out after the
 * call, or keep per slot which buffer holds its latest window and gather the
 * windows of the next call's slots into the buffer passed as state_in. The
 * delta state is updated in place and needs no such care.
 * Errors: those of gdn_decode_step; NULL (conv pointers), UNSUPPORTED (K),
 * ALIGN (conv buffers), SHAPE (state_out overlapping state_in).
 * ------------------------------------------------------------------------- */
gdn_status gdn_decode_layer(const gdn_dims *dims, int32_t batch, int32_t tokens_per_seq,
                            const gdn_conv_args *conv, const gdn_inputs *in, float *state,
                            const int32_t *state_slots, int32_t num_slots, int32_t out_dtype,
                            void *out, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_prefill_workspace_bytes -- device workspace gdn_prefill_chunked needs for
 * at most num_seqs sequences and total_tokens packed tokens (an upper bound
 * over every split of total_tokens into num_seqs lengths). Returns 0 when the
 * arguments are invalid.
 * ------------------------------------------------------------------------- */
size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int32_t num_seqs, int32_t total_tokens);

/* ---------------------------------------------------------------------------
 * gdn_prefill_chunked -- the same recurrence over packed variable-length
 * sequences, computed chunk-parallel (64-token chunks -- 32 when dk = 256 --
 * that start at each sequence's first token and never straddle two
 * sequences). Each path runs a kernel parallel over (chunk, k-head) that forms
 * the chunk's own quantities, then a carry per (sequence, v-head, slice of dv
 * rows) that runs the state-dependent products chunk after chunk. dk = dv = 128
 * takes f16 MFMA operands; the other head shapes keep f32 accuracy (f32 MFMA,
 * and bf16 hi/lo operand pairs on bf16 MFMA in the carry). The result equals
 * the token-by-token recurrence up to rounding order (ferrox-core src/gdn.rs
 * module doc: the chunked form is the same recurrence summed in another order;
 * ferrum-kernels tests page, `chunked_c64_matches_recurrent_oracle_and_
 * non_aligned_state_continuity`).
 *
 *   num_seqs         N >= 0
 *   cu_seqlens_host  host int32 [N+1] (validated: cu[0] = 0, non-decreasing,
 *                    cu[N] = total_tokens)
 *   cu_seqlens_dev   device int32 [N+1], the same values
 *   in               activations indexed by packed token row
 *   state            [N][Hv][dv][dk] f32: initial state in, final state out
 *   out_dtype, out   [total_tokens][Hv][dv]
 *   workspace        device, >= gdn_prefill_workspace_bytes(dims, N, total_tokens),
 *                    256-byte aligned; contents are scratch
 * Errors: NULL, SHAPE, UNSUPPORTED, OVERFLOW, ALIGN, WORKSPACE, LAUNCH.
 * ------------------------------------------------------------------------- */
gdn_status gdn_prefill_chunked(const gdn_dims *dims, int32_t num_seqs,
                               const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                               int32_t total_tokens, const gdn_inputs *in, float *state,
                               int32_t out_dtype, void *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_prefill_chunked_noalloc -- gdn_prefill_chunked for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * workspace in a static device array of the library instead of a caller buffer.
 *
 * Arguments and errors are those of gdn_prefill_chunked without the workspace.
 * The call allocates nothing. The array holds GDN_NOALLOC_SCRATCH_BYTES per GPU
 * (64 MiB: about 1,700 tokens of one sequence at Hk=16, Hv=32, dk=dv=128 without
 * the gated norm); a call whose gdn_prefill_workspace_bytes exceeds it returns
 * GDN_ERR_SCRATCH and launches nothing. Each GPU the library runs on holds its
 * own copy of the array until the process ends (its device address is looked
 * up on the first call on that device). Every call on one GPU shares that GPU's
 * copy and leaves its contents behind; nothing in it needs to start at zero.
 * Calls that overlap in time on one GPU (different streams, or different host
 * threads without ordering) race on the array: order them.
 * ------------------------------------------------------------------------- */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_chunked_noalloc(const gdn_dims *dims, int32_t num_seqs,
                                       const int32_t *cu_seqlens_host,
                                       const int32_t *cu_seqlens_dev, int32_t total_tokens,
                                       const gdn_inputs *in, float *state, int32_t out_dtype,
                                       void *out, void *stream);

/* ---------------------------------------------------------------------------
 * Kernel selection, for inspection and host-side tests. Which kernel a call runs
 * follows from its shape and from the device, as the ferrum-kernels tests page
 * checks for its own kernels (`chunk_k_gram_specialization_requires_repeated_
 * k128_heads`, `simd_delta_specialization_is_shape_and_device_capability_driven`).
 * These two calls report the choice the corresponding entry point makes, from the
 * same code; they make no HIP call and launch nothing.
 * ------------------------------------------------------------------------- */
typedef struct gdn_launch_info {
    int32_t waves;             /* decode: waves per workgroup */
    int32_t lanes_per_row;     /* decode: lanes holding one dk-wide state row */
    int32_t token_mode;        /* decode: 0 any token count, 1 token groups (fused layer,
                                  T > 1), 2 one token per sequence */
    int32_t nontemporal;       /* decode: 1 when GDN_STREAM_STATE selects the hinted kernel */
    int32_t carry_kind;        /* prefill: 0 split carry (compute + output wave per dv
                                  slice), 1 carry (one wave per slice); 2 the f32 carry
                                  of the head shapes other than 128 x 128 */
    int32_t slices_per_workgroup; /* prefill: 16-row dv slices per carry workgroup */
    int32_t workgroups;        /* grid of the decode kernel, or of the prefill carry */
    int32_t threads;           /* threads per workgroup of that kernel */
    int32_t prep_workgroups;   /* prefill: grid of the per-chunk preparation kernel */
} gdn_launch_info;

/* The decode kernel gdn_decode_step (fused_conv = 0) or gdn_decode_layer
 * (fused_conv = 1) runs for these dims (flags included), batch and tokens_per_seq.
 * Errors: NULL, SHAPE, UNSUPPORTED, as the entry points report them. */
gdn_status gdn_decode_launch_info(const gdn_dims *dims, int32_t batch, int32_t tokens_per_seq,
                                  int32_t fused_conv, gdn_launch_info *info);

/* The kernels gdn_prefill_chunked runs for these dims and sequences on a device
 * with `compute_units` CUs (the entry point queries the current device's count).
 * cu_seqlens_host: host int32 [N+1]. Errors: NULL, SHAPE, UNSUPPORTED. */
gdn_status gdn_prefill_launch_info(const gdn_dims *dims, int32_t num_seqs,
                                   const int32_t *cu_seqlens_host, int32_t total_tokens,
                                   int32_t compute_units, gdn_launch_info *info);

/* Static, NUL-terminated description of a status code. */
const char *gdn_status_string(gdn_status status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
