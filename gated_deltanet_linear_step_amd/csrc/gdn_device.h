// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn.so:
// activation dtype conversion, wave-level DPP reductions, gate activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum : uint32_t { F_L2NORM = 1u, F_RAW_GATES = 2u, F_GATED_NORM = 4u };

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

__device__ __forceinline__ float dot4(float4 a, float4 b)
{
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
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
