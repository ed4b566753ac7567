// Device helpers shared by the gfx950 kernels: element loads, wave64 lane
// exchanges (DPP and ds_swizzle), group reductions and the register-resident
// Walsh-Hadamard transform.
//
// Layout convention for one d-vector: a group of LPV = d/8 consecutive lanes
// of a wave64, lane gl (0 <= gl < LPV) holding elements [8*gl, 8*gl + 8).
// The transform H (Sylvester order, H[i][j] = (-1)^popcount(i&j)) is applied
// as log2(d) butterfly stages: the three stages on element bits 0..2 stay
// inside a lane, the stages on element bits 3.. exchange with lane gl ^ M
// (M = 1, 2, 4, ...).  "Butterfly WHT" is how the llama.cpp fork's README
// ("TurboQuant KV 캐시 압축 for llama.cpp", v1.7.0 "핵심 설계 결정" item 4)
// describes the encoder's rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqd {

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------
// Lane exchange: value of lane (lane ^ M).  M = 1, 2 and 8 are single DPP
// moves (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:8 inside a row of
// 16 lanes); M = 4 is two DPP moves (reverse the quad, then mirror the half
// row: lane i reads i^3^7 = i^4); M = 16 uses ds_swizzle in bitmask mode
// (xor_mask 16 over 32-lane halves); M = 32 uses ds_bpermute.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    const int x = __float_as_int(v);
    if constexpr (M == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));
    } else if constexpr (M == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));
    } else if constexpr (M == 4) {
        const int r = __builtin_amdgcn_update_dpp(0, x, 0x1B, 0xF, 0xF, true);
        return __int_as_float(__builtin_amdgcn_update_dpp(0, r, 0x141, 0xF, 0xF, true));
    } else if constexpr (M == 8) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true));
    } else if constexpr (M == 16) {
        return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
    } else {
        static_assert(M == 32, "xor distance");
        const int lane = __lane_id();
        return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, x));
    }
}

template <int M>
__device__ __forceinline__ uint32_t xor_lane_u(uint32_t v) {
    return as_u(xor_lane<M>(as_f(v)));
}

// Broadcast lane k of each quad to the whole quad (DPP quad_perm [k,k,k,k]).
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, K * 0x55, 0xF, 0xF, true);
}

// Sum over a group of LPV lanes (LPV a power of two <= 64).  Every lane of the
// group ends with the same bits: each stage adds the same two values in both
// partner lanes and float addition is commutative.
template <int LPV>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPV >= 2) v += xor_lane<1>(v);
    if constexpr (LPV >= 4) v += xor_lane<2>(v);
    if constexpr (LPV >= 8) v += xor_lane<4>(v);
    if constexpr (LPV >= 16) v += xor_lane<8>(v);
    if constexpr (LPV >= 32) v += xor_lane<16>(v);
    if constexpr (LPV >= 64) v += xor_lane<32>(v);
    return v;
}

template <int LPV>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (LPV >= 2) v = fmaxf(v, xor_lane<1>(v));
    if constexpr (LPV >= 4) v = fmaxf(v, xor_lane<2>(v));
    if constexpr (LPV >= 8) v = fmaxf(v, xor_lane<4>(v));
    if constexpr (LPV >= 16) v = fmaxf(v, xor_lane<8>(v));
    if constexpr (LPV >= 32) v = fmaxf(v, xor_lane<16>(v));
    if constexpr (LPV >= 64) v = fmaxf(v, xor_lane<32>(v));
    return v;
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard transform of a d = 8*LPV vector spread over a lane group.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ void cross_stage(float (&v)[8], int gl) {
    // partner lane holds the element whose index differs in bit log2(M)+3;
    // the lane with that bit clear keeps a + b, the other keeps a - b.
    const float sg = (gl & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = xor_lane<M>(v[e]);
        v[e] = fmaf(sg, v[e], p);
    }
}

template <int LPV>
__device__ __forceinline__ void fwht(float (&v)[8], int gl) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
        }
    }
    if constexpr (LPV >= 2) cross_stage<1>(v, gl);
    if constexpr (LPV >= 4) cross_stage<2>(v, gl);
    if constexpr (LPV >= 8) cross_stage<4>(v, gl);
    if constexpr (LPV >= 16) cross_stage<8>(v, gl);
    if constexpr (LPV >= 32) cross_stage<16>(v, gl);
}

// ---------------------------------------------------------------------------
// Element loads: 8 consecutive elements of type DT (0 f32, 1 f16, 2 bf16).
// `p` must be 16-byte aligned.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}

template <int DT>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
    if constexpr (DT == 0) {
        const float4* q = reinterpret_cast<const float4*>(p);
        const float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 r = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == 1) {
                v[2 * k] = half_bits_to_float(w[k] & 0xFFFFu);
                v[2 * k + 1] = half_bits_to_float(w[k] >> 16);
            } else {
                v[2 * k] = as_f(w[k] << 16);
                v[2 * k + 1] = as_f(w[k] & 0xFFFF0000u);
            }
        }
    }
}

template <int DT>
constexpr int elem_bytes() { return DT == 0 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Streaming loads for data read once (packed cache rows):
// non-temporal, so they do not displace reused data in the caches.  On MI355X
// a read-only stream with these loads reads about 8% faster than with plain
// ones.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream4(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint2 ld_stream2(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
    return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ uint32_t ld_stream1(const void* p) {
    return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

__device__ __forceinline__ uint32_t ld_stream_u16(const void* p) {
    return (uint32_t)__builtin_nontemporal_load(static_cast<const uint16_t*>(p));
}

// Half norm: clamp to the largest finite half, then round to nearest even.
__device__ __forceinline__ uint16_t norm_to_half(float n) {
    return float_to_half_bits(fminf(n, 65504.0f));
}

}  // namespace tqd
