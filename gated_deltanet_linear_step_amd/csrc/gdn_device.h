// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn.so:
// activation dtype conversion, wave-level DPP reductions, gate activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum : uint32_t { F_L2NORM = 1u, F_RAW_GATES = 2u, F_GATED_NORM = 4u, F_STREAM_STATE = 8u };

// ---- 16-bit float conversions (round to nearest even) ------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);  // keep NaN a (quiet) NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    _Float16 x;
    uint16_t b = (uint16_t)h;
    __builtin_memcpy(&x, &b, 2);
    return (float)x;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    _Float16 x = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &x, 2);
    return b;
}

// One activation element of dtype `dt` at element index idx.
__device__ __forceinline__ float load_act(const void *p, int64_t idx, int dt)
{
    if (dt == DT_F32)
        return static_cast<const float *>(p)[idx];
    uint32_t h = static_cast<const uint16_t *>(p)[idx];
    return dt == DT_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// Four consecutive activations starting at idx (idx % 4 == 0 and the base
// pointer aligned to 4 elements: the host checks both).
__device__ __forceinline__ float4 load_act4(const void *p, int64_t idx, int dt)
{
    if (dt == DT_F32)
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
    uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
    if (dt == DT_BF16)
        return make_float4(bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                           bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16));
    return make_float4(f16_bits_to_f32(w.x & 0xffffu), f16_bits_to_f32(w.x >> 16),
                       f16_bits_to_f32(w.y & 0xffffu), f16_bits_to_f32(w.y >> 16));
}

// Compile-time-dtype loads for the hot paths: no branch sits between a load
// and the next one, so independent loads stay in flight together.
template <int DT>
__device__ __forceinline__ float load_act_t(const void *p, int64_t idx)
{
    if constexpr (DT == DT_F32)
        return static_cast<const float *>(p)[idx];
    const uint32_t h = static_cast<const uint16_t *>(p)[idx];
    if constexpr (DT == DT_BF16)
        return bf16_bits_to_f32(h);
    return f16_bits_to_f32(h);
}

template <int DT>
__device__ __forceinline__ float4 load_act4_t(const void *p, int64_t idx)
{
    if constexpr (DT == DT_F32)
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
    if constexpr (DT == DT_BF16)
        return make_float4(bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                           bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16));
    return make_float4(f16_bits_to_f32(w.x & 0xffffu), f16_bits_to_f32(w.x >> 16),
                       f16_bits_to_f32(w.y & 0xffffu), f16_bits_to_f32(w.y >> 16));
}

// A zero the compiler cannot see through, in a VGPR. Added to a workgroup-uniform
// element index it keeps that load on the vector memory path: as a scalar load it
// would need its own wait, which also holds back every vector load whose address
// comes from a scalar register loaded at the same time.
__device__ __forceinline__ int vgpr_zero()
{
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// One element of runtime dtype `dt`, read without a branch: the 32-bit word
// holding it is loaded (the base pointer is 4-byte aligned -- the host checks),
// then the conversion is selected. Split into the load and the conversion so a
// caller can issue other loads in between. Only for arrays read in runs of even
// length from an even element (z: [tokens][Hv][dv] with dv even in every built
// shape; q, k, v rows, 4-element aligned with even head dims), so the word of a
// 16-bit element never reaches past the run's last element.
__device__ __forceinline__ uint32_t load_word_nb(const void *p, int64_t idx, int dt)
{
    const int64_t byte = dt == DT_F32 ? idx * 4 : idx * 2;
    return *reinterpret_cast<const uint32_t *>(static_cast<const char *>(p) + (byte & ~(int64_t)3));
}

__device__ __forceinline__ float word_to_f32(uint32_t w, int64_t idx, int dt)
{
    const uint32_t h = (idx & 1) ? (w >> 16) : (w & 0xffffu);
    const float vf16 = f16_bits_to_f32(h), vbf16 = bf16_bits_to_f32(h);
    return dt == DT_F32 ? __uint_as_float(w) : (dt == DT_BF16 ? vbf16 : vf16);
}

// One gate input element (16-bit or f32) as two 16-bit loads that never leave the
// element (an f32 element's halves, or a 16-bit element read twice), so the load
// is issued without a branch on the dtype and never reads past the array's end;
// the two halves are kept packed in one register.
struct GateWord {
    uint32_t bits;
};
__device__ __forceinline__ GateWord load_gate(const void *p, int64_t idx, int dt)
{
    const uint16_t *b = static_cast<const uint16_t *>(p) + (dt == DT_F32 ? 2 * idx : idx);
    return GateWord{(uint32_t)b[0] | ((uint32_t)b[dt == DT_F32 ? 1 : 0] << 16)};
}
__device__ __forceinline__ float gate_value(GateWord w, int dt)
{
    const uint32_t lo = w.bits & 0xffffu;
    return dt == DT_F32 ? __uint_as_float(w.bits) : (dt == DT_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo));
}

// Raw bits of four consecutive activations of compile-time dtype DT (8 bytes for
// 16-bit types, 16 for f32) and their conversion.
template <int DT>
struct Raw4 {
    uint32_t w[DT == DT_F32 ? 4 : 2];
};

template <int DT>
__device__ __forceinline__ Raw4<DT> load_raw4(const void *p, int64_t idx)
{
    Raw4<DT> r;
    if constexpr (DT == DT_F32) {
        const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p) + idx);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}

template <int DT>
__device__ __forceinline__ float4 raw4_to_f32(const Raw4<DT> &r)
{
    if constexpr (DT == DT_F32)
        return make_float4(__uint_as_float(r.w[0]), __uint_as_float(r.w[1]),
                           __uint_as_float(r.w[2]), __uint_as_float(r.w[3]));
    else if constexpr (DT == DT_BF16)
        return make_float4(bf16_bits_to_f32(r.w[0] & 0xffffu), bf16_bits_to_f32(r.w[0] >> 16),
                           bf16_bits_to_f32(r.w[1] & 0xffffu), bf16_bits_to_f32(r.w[1] >> 16));
    else
        return make_float4(f16_bits_to_f32(r.w[0] & 0xffffu), f16_bits_to_f32(r.w[0] >> 16),
                           f16_bits_to_f32(r.w[1] & 0xffffu), f16_bits_to_f32(r.w[1] >> 16));
}

template <int DT>
__device__ __forceinline__ uint32_t load_raw1(const void *p, int64_t idx)
{
    if constexpr (DT == DT_F32)
        return static_cast<const uint32_t *>(p)[idx];
    else
        return static_cast<const uint16_t *>(p)[idx];
}

template <int DT>
__device__ __forceinline__ float raw1_to_f32(uint32_t w)
{
    if constexpr (DT == DT_F32)
        return __uint_as_float(w);
    else if constexpr (DT == DT_BF16)
        return bf16_bits_to_f32(w);
    else
        return f16_bits_to_f32(w);
}

__device__ __forceinline__ void store_act(void *p, int64_t idx, int dt, float v)
{
    if (dt == DT_F32)
        static_cast<float *>(p)[idx] = v;
    else if (dt == DT_BF16)
        static_cast<uint16_t *>(p)[idx] = f32_to_bf16_bits(v);
    else
        static_cast<uint16_t *>(p)[idx] = f32_to_f16_bits(v);
}

// ---- wave-level reductions ---------------------------------------------------
// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror
// (lane i <-> 7-i within 8), row_mirror (lane i <-> 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64); every
// lane of a group receives the group's sum. After the quad steps all lanes of a
// quad hold the quad sum, so the two mirrors pair each group with its neighbour.
template <int W>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (W >= 2)
        x += dpp_mov<0xB1>(x);
    if constexpr (W >= 4)
        x += dpp_mov<0x4E>(x);
    if constexpr (W >= 8)
        x += dpp_mov<0x141>(x);
    if constexpr (W >= 16)
        x += dpp_mov<0x140>(x);
    if constexpr (W >= 32)  // lane ^ 16 within each 32-lane half (ds_swizzle bit mode)
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    if constexpr (W >= 64)
        x += __shfl_xor(x, 32, 64);
    return x;
}

// An explicit fused chain: every kernel that calls it rounds the same way
__device__ __forceinline__ float dot4(float4 a, float4 b)
{
    return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

// ---- gate activations (split-by-sign sigmoid, softplus with +-20 cut-overs) ----
__device__ __forceinline__ float sigmoid_f(float x)
{
    if (x >= 0.f)
        return 1.f / (1.f + expf(-x));
    float e = expf(x);
    return e / (1.f + e);
}

__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

__device__ __forceinline__ float softplus_f(float x)
{
    if (x > 20.f)
        return x;
    if (x < -20.f)
        return expf(x);
    return log1pf(expf(x));
}

// k-head read by v-head h: grouped h / (Hv/Hk), tiled h % Hk.
__device__ __forceinline__ int k_head_of(int head_map, int h, int Hk, int Hv)
{
    return head_map == 0 ? h / (Hv / Hk) : h % Hk;
}

}  // namespace gdn
