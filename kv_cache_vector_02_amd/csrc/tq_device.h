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
    if constexpr (LPV >= 64) cross_stage<32>(v, gl);
}

// Second pass of the double transform S1 -> WHT -> S2 -> WHT ("TurboQuant KV
// 캐시 압축 for llama.cpp", v1.5.3 "핵심 변경" item 1) on a vector in the
// natural layout: v <- H(D3 v) / sqrt(d), D3 given by its sign bits (bit i =
// dim i).  After the first transform H(D x) this gives R D x with
// R = H D3 H / sqrt(d); R is symmetric, so the same pass after H also inverts.
template <int LPV>
__device__ __forceinline__ void second_pass(float (&v)[8], int gl, const uint32_t* mask3) {
    const uint32_t s3 = (mask3[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e]) ^ (((s3 >> e) & 1u) << 31));
    fwht<LPV>(v, gl);
    const float r = 1.0f / __builtin_sqrtf((float)(8 * LPV));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= r;
}

// ---------------------------------------------------------------------------
// The same transform with every cross-lane stage as one fused DPP
// multiply-add, y_l = x_l + c_l * x_{l ^ v} (v_fmac_f32 with the partner read
// through DPP), for the encoder, whose cost is its VALU instruction count.
// Partners l ^ 1, l ^ 2 (quad_perm), l ^ 7 (row_half_mirror), l ^ 8
// (row_ror:8), l ^ 16 (ds_swizzle) and l ^ 32 (ds_bpermute), with
// c_l = (-1)^popcount(l & w) for
// w = 5, 6, 4, 8, 16, 32.  Every stage keeps a + b in one lane of a pair and
// b - a (not a - b) in the other, and the partners are not the unit steps of
// the plain butterfly; the network still equals H, applied to the lane blocks
// in a fixed order: lane gl must hold the input elements of lane
// fwht_src_lane(gl) (their 8 elements in place) to receive H x in Sylvester
// order.  (Both facts are exact identities of the +-1 matrices, checked for
// every d by multiplying the stages out.)
// ---------------------------------------------------------------------------
template <int LPV>
__device__ __forceinline__ int fwht_src_lane(int gl) {
    static_assert(LPV == 4 || LPV == 8 || LPV == 16 || LPV == 32 || LPV == 64, "lane group of 4..64 lanes");
    if constexpr (LPV == 4) return gl ^ 3;
    // lanes 0..7 of each block of 8 read 7 2 1 4 0 5 6 3 (affine in the lane
    // bits); the blocks of 8 come in reverse order
    const int lo = (int)((0x36504127u >> (4 * (gl & 7))) & 7u);
    return lo | ((~gl) & (LPV - 1) & ~7);
}

template <int W>
__device__ __forceinline__ float parity_sign(int gl) {
    return (__builtin_popcount(gl & W) & 1) ? -1.0f : 1.0f;
}

// x[e] += c * x[e] of the DPP partner lane, for the 8 elements, as
// v_fmac_f32_dpp (one instruction each).  The compiler does not fold a DPP
// move into a multiply-add that overwrites the moved register, hence the asm;
// the leading s_nop 1 gives the two wait states a DPP read needs after a VALU
// write of its source (inside the block every source was written eight
// instructions earlier).  All lanes of the wave are active where it is used.
#define TQ_FMAC_DPP8(x, c, DPP)                                                                          \
    asm("s_nop 1\n"                                                                                      \
        "v_fmac_f32_dpp %0, %0, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %1, %1, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %2, %2, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %3, %3, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %4, %4, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %5, %5, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %6, %6, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"                    \
        "v_fmac_f32_dpp %7, %7, %8 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1"                      \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]) \
        : "v"(c))

template <int LPV>
__device__ __forceinline__ void fwht_fused(float (&v)[8], int gl) {
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
    const float c1 = parity_sign<5 & (LPV - 1)>(gl), c2 = parity_sign<6 & (LPV - 1)>(gl);
    TQ_FMAC_DPP8(v, c1, "quad_perm:[1,0,3,2]");  // l ^ 1
    TQ_FMAC_DPP8(v, c2, "quad_perm:[2,3,0,1]");  // l ^ 2
    if constexpr (LPV >= 8) {
        const float c3 = parity_sign<4>(gl);
        TQ_FMAC_DPP8(v, c3, "row_half_mirror");  // l ^ 7
    }
    if constexpr (LPV >= 16) {
        const float c4 = parity_sign<8>(gl);
        TQ_FMAC_DPP8(v, c4, "row_ror:8");  // l ^ 8
    }
    if constexpr (LPV >= 32) {
        const float c5 = parity_sign<16>(gl);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(xor_lane<16>(v[e]), c5, v[e]);  // l ^ 16
    }
    if constexpr (LPV >= 64) {
        const float c6 = parity_sign<32>(gl);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(xor_lane<32>(v[e]), c6, v[e]);  // l ^ 32
    }
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

// The raw bits of 8 elements: two 16-byte words for f32, one for f16/bf16.
template <int DT>
struct Raw8 {
    uint4 w[DT == 0 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float (&v)[8]) {
    if constexpr (DT == 0) {
        v[0] = as_f(r.w[0].x); v[1] = as_f(r.w[0].y); v[2] = as_f(r.w[0].z); v[3] = as_f(r.w[0].w);
        v[4] = as_f(r.w[1].x); v[5] = as_f(r.w[1].y); v[6] = as_f(r.w[1].z); v[7] = as_f(r.w[1].w);
    } else {
        const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
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
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
    Raw8<DT> r;
#pragma unroll
    for (int k = 0; k < (DT == 0 ? 2 : 1); ++k) r.w[k] = reinterpret_cast<const uint4*>(p)[k];
    unpack8<DT>(r, v);
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

// 8 elements of type DT read once (non-temporal); `p` 16-byte aligned.
template <int DT>
__device__ __forceinline__ void ld_stream8(const void* p, Raw8<DT>& r) {
#pragma unroll
    for (int k = 0; k < (DT == 0 ? 2 : 1); ++k) r.w[k] = ld_stream4(static_cast<const uint4*>(p) + k);
}

// Half norm: clamp to the largest finite half, then round to nearest even.
__device__ __forceinline__ uint16_t norm_to_half(float n) {
    return float_to_half_bits(fminf(n, 65504.0f));
}

}  // namespace tqd
