// gdn_api.cpp -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Every entry point validates all of its arguments on the host before the first
// HIP call, so a call that returns an error has launched nothing and changed
// no buffer. Only GDN_ERR_LAUNCH is reported after a launch was attempted.

#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "gdn_kernels.h"

namespace {

constexpr uint32_t kPrefillFlags = GDN_L2NORM_QK | GDN_RAW_GATES | GDN_GATED_NORM;
constexpr uint32_t kDecodeFlags = kPrefillFlags | GDN_STREAM_STATE;
constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

bool dtype_ok(int32_t dt) { return dt == GDN_F32 || dt == GDN_F16 || dt == GDN_BF16; }
int64_t dtype_size(int32_t dt) { return dt == GDN_F32 ? 4 : 2; }

bool aligned(const void *p, int64_t bytes)
{
    return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes)) == 0;
}

// Checks shared by the decode step and the prefill: dims, flags and the inputs
// the flags require. On success fills the kernel-side copies.
gdn_status check_common(const gdn_dims *d, const gdn_inputs *in, int32_t out_dtype,
                        const void *out, const float *state, bool (*supported)(int, int),
                        uint32_t known_flags, gdn::HeadCfg &hc, gdn::ActInputs &ai)
{
    if (!d || !in || !out || !state)
        return GDN_ERR_NULL;
    if (d->num_k_heads < 1 || d->num_v_heads < 1 || d->num_v_heads % d->num_k_heads != 0)
        return GDN_ERR_SHAPE;
    if (d->head_dim_k < 1 || d->head_dim_v < 1)
        return GDN_ERR_SHAPE;
    if (d->head_map != GDN_MAP_GROUPED && d->head_map != GDN_MAP_TILED)
        return GDN_ERR_SHAPE;
    if ((d->flags & ~known_flags) != 0)
        return GDN_ERR_UNSUPPORTED;
    if (!supported(d->head_dim_k, d->head_dim_v))
        return GDN_ERR_UNSUPPORTED;
    if (!(std::isfinite(d->scale) && std::isfinite(d->l2_eps) && std::isfinite(d->norm_eps)) ||
        d->scale < 0.f || d->l2_eps < 0.f || d->norm_eps < 0.f)
        return GDN_ERR_SHAPE;
    if (!dtype_ok(out_dtype) || !dtype_ok(in->qkv_dtype))
        return GDN_ERR_UNSUPPORTED;
    if (!in->q || !in->k || !in->v)
        return GDN_ERR_NULL;
    const int64_t qk_w = (int64_t)d->num_k_heads * d->head_dim_k;
    const int64_t v_w = (int64_t)d->num_v_heads * d->head_dim_v;
    if (in->q_stride < qk_w || in->k_stride < qk_w || in->v_stride < v_w)
        return GDN_ERR_SHAPE;
    // q, k and v are read as groups of 4 elements: base and row stride must keep
    // every group aligned to 4 elements.
    const int64_t es = dtype_size(in->qkv_dtype);
    if (!aligned(in->q, 4 * es) || !aligned(in->k, 4 * es) || !aligned(in->v, 4 * es) ||
        in->q_stride % 4 != 0 || in->k_stride % 4 != 0 || in->v_stride % 4 != 0)
        return GDN_ERR_ALIGN;
    if (d->flags & GDN_RAW_GATES) {
        if (!in->a || !in->b || !in->decay_param || !in->dt_bias)
            return GDN_ERR_NULL;
        if (!dtype_ok(in->ab_dtype))
            return GDN_ERR_UNSUPPORTED;
        if (d->decay != GDN_DECAY_LOG_RATE && d->decay != GDN_DECAY_NEGATIVE_RATE)
            return GDN_ERR_SHAPE;
        const int64_t gs = dtype_size(in->ab_dtype);
        if (!aligned(in->a, gs) || !aligned(in->b, gs))
            return GDN_ERR_ALIGN;  // gate elements are read whole, never past the last one
    } else if (!in->g || !in->beta) {
        return GDN_ERR_NULL;
    } else if (!aligned(in->g, 4) || !aligned(in->beta, 4)) {
        return GDN_ERR_ALIGN;
    }
    if (d->flags & GDN_GATED_NORM) {
        if (!in->z || !in->norm_weight)
            return GDN_ERR_NULL;
        if (!dtype_ok(in->z_dtype))
            return GDN_ERR_UNSUPPORTED;
        if (!aligned(in->z, 4) || !aligned(in->norm_weight, 4))
            return GDN_ERR_ALIGN;  // z is read as aligned 32-bit words
    }
    if (!aligned(state, 16))
        return GDN_ERR_ALIGN;

    hc.Hk = d->num_k_heads;
    hc.Hv = d->num_v_heads;
    hc.dk = d->head_dim_k;
    hc.dv = d->head_dim_v;
    hc.head_map = d->head_map;
    hc.decay_kind = d->decay;
    hc.flags = d->flags;
    hc.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->head_dim_k);
    hc.l2_eps = d->l2_eps > 0.f ? d->l2_eps : 1e-6f;
    hc.norm_eps = d->norm_eps > 0.f ? d->norm_eps : 1e-6f;

    ai.q = in->q;
    ai.k = in->k;
    ai.v = in->v;
    ai.q_stride = in->q_stride;
    ai.k_stride = in->k_stride;
    ai.v_stride = in->v_stride;
    ai.qkv_dt = in->qkv_dtype;
    ai.a = in->a;
    ai.b = in->b;
    ai.ab_dt = in->ab_dtype;
    ai.decay_param = in->decay_param;
    ai.dt_bias = in->dt_bias;
    ai.g = in->g;
    ai.beta = in->beta;
    ai.z = in->z;
    ai.z_dt = in->z_dtype;
    ai.norm_w = in->norm_weight;
    return GDN_OK;
}

gdn_status launch_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// Validates host cu_seqlens; fills the chunk counts (chunks of `clen` tokens) the
// prefill grid needs.
gdn_status check_cu(const int32_t *cu, int32_t n, int32_t total, int clen, int64_t *chunks,
                    int64_t *max_chunks)
{
    if (cu[0] != 0 || cu[n] != total)
        return GDN_ERR_SHAPE;
    int64_t c = 0, mx = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (cu[i + 1] < cu[i])
            return GDN_ERR_SHAPE;
        const int64_t ci = ((int64_t)cu[i + 1] - cu[i] + clen - 1) / clen;
        c += ci;
        if (ci > mx)
            mx = ci;
    }
    *chunks = c;
    *max_chunks = mx;
    return GDN_OK;
}

// An upper bound on a call's chunk count over every split of total_tokens into
// num_seqs sequences: total / chunk length + one partial chunk per sequence.
int64_t max_chunk_bound(const gdn_dims *d, int32_t num_seqs, int32_t total_tokens)
{
    return (int64_t)total_tokens / gdn::prefill_chunk_len(d->head_dim_k, d->head_dim_v) + num_seqs;
}

// Everything gdn_prefill_chunked checks except the workspace; fills the kernel
// parameters, the workspace the call needs, and whether it has no tokens at all.
gdn_status prefill_prepare(const gdn_dims *dims, int32_t num_seqs, const int32_t *cu_seqlens_host,
                           const int32_t *cu_seqlens_dev, int32_t total_tokens, const gdn_inputs *in,
                           float *state, int32_t out_dtype, void *out, gdn::PrefillParams &p,
                           size_t &need, bool &empty)
{
    gdn_status st = check_common(dims, in, out_dtype, out, state, gdn::prefill_supported, kPrefillFlags,
                                 p.hc, p.in);
    if (st != GDN_OK)
        return st;
    if (num_seqs < 0 || total_tokens < 0)
        return GDN_ERR_SHAPE;
    if (!cu_seqlens_host || !cu_seqlens_dev)
        return GDN_ERR_NULL;
    empty = total_tokens == 0;
    if (num_seqs == 0)
        return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
    int64_t chunks = 0, max_chunks = 0;
    const int clen = gdn::prefill_chunk_len(dims->head_dim_k, dims->head_dim_v);
    st = check_cu(cu_seqlens_host, num_seqs, total_tokens, clen, &chunks, &max_chunks);
    if (st != GDN_OK)
        return st;
    if ((int64_t)total_tokens * dims->num_v_heads > kI32Max || chunks * dims->num_v_heads > kI32Max)
        return GDN_ERR_OVERFLOW;
    const int64_t mc = (int64_t)total_tokens / clen + num_seqs;
    need = gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_dim_k,
                                        dims->head_dim_v, mc, num_seqs, total_tokens,
                                        (dims->flags & GDN_GATED_NORM) != 0);
    p.state = state;
    p.out = out;
    p.out_dt = out_dtype;
    p.N = num_seqs;
    p.total = total_tokens;
    p.cu = cu_seqlens_dev;
    p.num_chunks = (int)chunks;
    p.max_seq_chunks = (int)max_chunks;
    return GDN_OK;
}

// ---- the static scratch of gdn_prefill_chunked_noalloc ----------------------
// The prefill's workspace for callers that cannot allocate (graph capture, tight
// serving loops): a file-scope device array, one copy per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, never device
// memory: its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void **addr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = p;
    }
    *addr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "inconsistent sizes or sequence offsets";
    case GDN_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case GDN_ERR_OVERFLOW: return "an element count or offset exceeds the kernels' index range";
    case GDN_ERR_ALIGN: return "a pointer or stride is not aligned as required";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case GDN_ERR_SCRATCH: return "the call needs more than the no-allocation entry point's static scratch";
    }
    return "unknown status";
}

int32_t gdn_version(void) { return 200; }

gdn_status gdn_decode_launch_info(const gdn_dims *d, int32_t batch, int32_t tokens_per_seq,
                                  int32_t fused_conv, gdn_launch_info *info)
{
    if (!d || !info)
        return GDN_ERR_NULL;
    if (d->num_k_heads < 1 || d->num_v_heads < 1 || d->num_v_heads % d->num_k_heads != 0 ||
        batch < 0 || tokens_per_seq < 1)
        return GDN_ERR_SHAPE;
    if ((d->flags & ~kDecodeFlags) != 0 || !gdn::decode_supported(d->head_dim_k, d->head_dim_v))
        return GDN_ERR_UNSUPPORTED;
    const gdn::DecodePlan pl = gdn::decode_plan(d->head_dim_k, d->head_dim_v, batch, tokens_per_seq,
                                                d->num_v_heads, fused_conv != 0, d->flags);
    *info = gdn_launch_info{};
    info->waves = pl.waves;
    info->lanes_per_row = pl.lanes_per_row;
    info->token_mode = pl.mode;
    info->nontemporal = pl.nontemporal;
    info->workgroups = pl.workgroups;
    info->threads = pl.threads;
    return GDN_OK;
}

gdn_status gdn_prefill_launch_info(const gdn_dims *d, int32_t num_seqs, const int32_t *cu_seqlens_host,
                                   int32_t total_tokens, int32_t compute_units, gdn_launch_info *info)
{
    if (!d || !info || !cu_seqlens_host)
        return GDN_ERR_NULL;
    if (d->num_k_heads < 1 || d->num_v_heads < 1 || d->num_v_heads % d->num_k_heads != 0 ||
        num_seqs < 1 || total_tokens < 0 || compute_units < 1)
        return GDN_ERR_SHAPE;
    if ((d->flags & ~kPrefillFlags) != 0 || !gdn::prefill_supported(d->head_dim_k, d->head_dim_v))
        return GDN_ERR_UNSUPPORTED;
    int64_t chunks = 0, max_chunks = 0;
    const gdn_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens,
                                   gdn::prefill_chunk_len(d->head_dim_k, d->head_dim_v), &chunks,
                                   &max_chunks);
    if (st != GDN_OK)
        return st;
    const gdn::PrefillPlan pl = gdn::prefill_plan(num_seqs, d->num_k_heads, d->num_v_heads,
                                                  d->head_dim_k, d->head_dim_v, chunks, compute_units);
    *info = gdn_launch_info{};
    info->carry_kind = pl.carry_kind;
    info->slices_per_workgroup = pl.slices_per_wg;
    info->workgroups = pl.carry_workgroups;
    info->threads = pl.carry_threads;
    info->prep_workgroups = pl.prep_workgroups;
    return GDN_OK;
}

gdn_status gdn_conv_update(int32_t channels, int32_t kernel_size, int32_t num_seqs,
                           const int32_t *cu_seqlens, int32_t total_tokens, int32_t x_dtype,
                           const void *x, int64_t x_stride, const void *weight, void *conv_state,
                           int32_t y_dtype, void *y, int64_t y_stride, void *stream)
{
    if (channels < 1 || num_seqs < 0 || total_tokens < 0)
        return GDN_ERR_SHAPE;
    if (kernel_size < 2 || kernel_size > 8)
        return GDN_ERR_UNSUPPORTED;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype))
        return GDN_ERR_UNSUPPORTED;
    if (total_tokens > 0 && num_seqs == 0)
        return GDN_ERR_SHAPE;
    if (num_seqs == 0 || total_tokens == 0)
        return GDN_OK;  // nothing to do; states untouched
    if (!x || !weight || !conv_state || !y)
        return GDN_ERR_NULL;
    if (x_stride < channels || y_stride < channels)
        return GDN_ERR_SHAPE;
    if (!cu_seqlens && total_tokens % num_seqs != 0)
        return GDN_ERR_SHAPE;
    const int64_t cblocks = ((int64_t)channels + 255) / 256;
    if (cblocks * total_tokens > kI32Max)
        return GDN_ERR_OVERFLOW;
    gdn::ConvParams p{};
    p.C = channels;
    p.K = kernel_size;
    p.N = num_seqs;
    p.total = total_tokens;
    p.uniform_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    p.cu = cu_seqlens;
    p.x = x;
    p.x_stride = x_stride;
    p.w = weight;
    p.state = conv_state;
    p.y = y;
    p.y_stride = y_stride;
    p.x_dt = x_dtype;
    p.y_dt = y_dtype;
    return launch_status(gdn::launch_conv(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_step(const gdn_dims *dims, int32_t batch, int32_t tokens_per_seq,
                           const gdn_inputs *in, float *state, const int32_t *state_slots,
                           int32_t num_slots, int32_t out_dtype, void *out, void *stream)
{
    gdn::DecodeParams p{};
    gdn_status st = check_common(dims, in, out_dtype, out, state, gdn::decode_supported, kDecodeFlags,
                                 p.hc, p.in);
    if (st != GDN_OK)
        return st;
    if (batch < 0 || tokens_per_seq < 1 || num_slots < 0)
        return GDN_ERR_SHAPE;
    if (!state_slots && num_slots < batch)
        return GDN_ERR_SHAPE;
    if ((int64_t)batch * tokens_per_seq > kI32Max || (int64_t)batch * dims->num_v_heads > kI32Max)
        return GDN_ERR_OVERFLOW;
    if (batch == 0)
        return GDN_OK;
    p.state = state;
    p.slots = state_slots;
    p.num_slots = num_slots;
    p.out = out;
    p.out_dt = out_dtype;
    p.B = batch;
    p.T = tokens_per_seq;
    return launch_status(gdn::launch_decode(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_layer(const gdn_dims *dims, int32_t batch, int32_t tokens_per_seq,
                            const gdn_conv_args *conv, const gdn_inputs *in, float *state,
                            const int32_t *state_slots, int32_t num_slots, int32_t out_dtype,
                            void *out, void *stream)
{
    gdn::DecodeParams p{};
    gdn_status st = check_common(dims, in, out_dtype, out, state, gdn::decode_supported, kDecodeFlags,
                                 p.hc, p.in);
    if (st != GDN_OK)
        return st;
    if (!conv || !conv->weight || !conv->state_in || !conv->state_out)
        return GDN_ERR_NULL;
    if (conv->kernel_size != 4)
        return GDN_ERR_UNSUPPORTED;  // the built conv width
    if (batch < 0 || tokens_per_seq < 1 || num_slots < 0)
        return GDN_ERR_SHAPE;
    if (!state_slots && num_slots < batch)
        return GDN_ERR_SHAPE;
    if ((int64_t)batch * tokens_per_seq > kI32Max || (int64_t)batch * dims->num_v_heads > kI32Max)
        return GDN_ERR_OVERFLOW;
    const int64_t es = dtype_size(in->qkv_dtype);
    if (!aligned(conv->weight, 4 * es) || !aligned(conv->state_in, 4 * es) ||
        !aligned(conv->state_out, 4 * es))
        return GDN_ERR_ALIGN;
    // the new window goes to a second buffer (the q/k channels of a k-head are
    // read by several workgroups), so the two may not overlap
    const int64_t channels = 2 * (int64_t)dims->num_k_heads * dims->head_dim_k +
                             (int64_t)dims->num_v_heads * dims->head_dim_v;
    const int64_t sbytes = (int64_t)num_slots * channels * (conv->kernel_size - 1) * es;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(conv->state_in);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(conv->state_out);
    if (sbytes > 0 && a0 < b0 + (uintptr_t)sbytes && b0 < a0 + (uintptr_t)sbytes)
        return GDN_ERR_SHAPE;
    if (batch == 0)
        return GDN_OK;
    p.state = state;
    p.slots = state_slots;
    p.num_slots = num_slots;
    p.out = out;
    p.out_dt = out_dtype;
    p.B = batch;
    p.T = tokens_per_seq;
    p.conv_k = conv->kernel_size;
    p.conv_w = conv->weight;
    p.conv_in = conv->state_in;
    p.conv_out = conv->state_out;
    return launch_status(gdn::launch_decode(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(const gdn_dims *d, int32_t num_seqs, int32_t total_tokens)
{
    if (!d || num_seqs < 0 || total_tokens < 0 || d->num_k_heads < 1 || d->num_v_heads < 1 ||
        d->num_v_heads % d->num_k_heads != 0 || !gdn::prefill_supported(d->head_dim_k, d->head_dim_v))
        return 0;
    const int64_t max_chunks = max_chunk_bound(d, num_seqs, total_tokens);
    return gdn::prefill_workspace_bytes(d->num_k_heads, d->num_v_heads, d->head_dim_k,
                                        d->head_dim_v, max_chunks, num_seqs, total_tokens,
                                        (d->flags & GDN_GATED_NORM) != 0);
}

gdn_status gdn_prefill_chunked(const gdn_dims *dims, int32_t num_seqs,
                               const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                               int32_t total_tokens, const gdn_inputs *in, float *state,
                               int32_t out_dtype, void *out, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    gdn::PrefillParams p{};
    size_t need = 0;
    bool empty = false;
    gdn_status st = prefill_prepare(dims, num_seqs, cu_seqlens_host, cu_seqlens_dev, total_tokens, in,
                                    state, out_dtype, out, p, need, empty);
    if (st != GDN_OK || (empty && num_seqs == 0))
        return st;
    if (!workspace || workspace_bytes < need)
        return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return GDN_ERR_ALIGN;
    if (empty)
        return GDN_OK;  // every sequence empty: states untouched
    gdn::prefill_carve(p, workspace, max_chunk_bound(dims, num_seqs, total_tokens));
    return launch_status(gdn::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_dims *dims, int32_t num_seqs,
                                       const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                                       int32_t total_tokens, const gdn_inputs *in, float *state,
                                       int32_t out_dtype, void *out, void *stream)
{
    gdn::PrefillParams p{};
    size_t need = 0;
    bool empty = false;
    gdn_status st = prefill_prepare(dims, num_seqs, cu_seqlens_host, cu_seqlens_dev, total_tokens, in,
                                    state, out_dtype, out, p, need, empty);
    if (st != GDN_OK || empty)
        return st;
    if (need > kScratchBytes)
        return GDN_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess)
        return GDN_ERR_LAUNCH;
    gdn::prefill_carve(p, ws, max_chunk_bound(dims, num_seqs, total_tokens));
    return launch_status(gdn::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
