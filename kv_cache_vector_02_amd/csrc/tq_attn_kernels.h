// Decode attention over the packed cache, gfx950, float32 VALU.
//
// Three launches per call:
//   1. qprep: q_rot = H(D_K q) per query head (register/DPP transform), stored
//      pre-scaled by scale*log2(e)/d; with QJL also S q_rot/sqrt(d).
//   2. split: grid (splits, kv_head x head_chunk, batch).  Each wave streams
//      64-token tiles of its split: lane <-> token for the K side (codes in
//      registers, centroid pairs from an LDS table, rotated query from scalar
//      registers), a wave-wide online softmax in the log2 domain, then lane <->
//      dimension pairs for the V side (codes staged in LDS, softmax weights
//      broadcast from LDS), accumulating V in the rotated domain.  The four
//      waves of a block merge their (max, sum, acc) and write one partial.
//   3. combine: log-sum-exp merge of the partials of each (batch, head), one
//      inverse transform D_V H(.)/d per output head.
//
// The method is the one described by "TurboQuant KV 캐시 압축 for llama.cpp":
// Q-side WHT so the rotation cancels (v1.7.0 "핵심 설계 결정" item 4), float (not
// half2) accumulation of the V sum (v1.5.2 "핵심 변경" items 1-2), V summed in the
// rotated domain with one inverse transform per output (v1.5.1 item 2), and the
// QJL scalar correction read from the raw K block (v1.4.2 items 2 and 5).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include <utility>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace attn {

using namespace tqd;

template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr float kLog2e = 1.4426950408889634f;

// Waves per SIMD the split kernel is compiled for (caps its VGPRs at 512/N).
#ifndef TQ_SPLIT_WAVES
#define TQ_SPLIT_WAVES(D) ((D) == 128 ? 3 : 2)
#endif

// ----------------------------------------------------------------- qprep ----
// q_rot is stored dim-major inside each chunk of G query heads, so the 2*G
// values one K lookup needs are contiguous for the scalar loads.
template <int D, int DT>
__global__ __launch_bounds__(64) void qprep_kernel(AttnArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    __shared__ float rot[VPW][D];
    const int lane = threadIdx.x;
    const int gl = lane & (LPV - 1), grp = lane / LPV;
    const int heads = a.batch * a.hq;
    const int head = blockIdx.x * VPW + grp;
    const bool valid = head < heads;
    const uint32_t sbits = (a.kc.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
    float v[8];
    if (valid) {
        const char* p = static_cast<const char*>(a.q) + ((int64_t)head * D + gl * 8) * elem_bytes<DT>();
        load8<DT>(p, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e]) ^ (((sbits >> e) & 1u) << 31));
    fwht<LPV>(v, gl);
    const float qs = a.scale * kLog2e / (float)D;
    if (valid) {
        // dim-major inside each chunk of G heads: [head - hh][dim][hh]
        const int G = a.heads_per_chunk;
        const int hh = head % G;
        float* o = a.qrot + (int64_t)(head - hh) * D + hh;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[(gl * 8 + e) * G] = v[e] * qs;
    }
    const int m = a.kc.qjl_m;
    if (m > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rot[grp][gl * 8 + e] = v[e];
        __syncthreads();
        const float ps = a.scale * kLog2e * sqrtf(1.57079632679489662f) / ((float)m * sqrtf((float)D));
        for (int j = gl; j < m; j += LPV) {
            const float* srow = a.S + (int64_t)j * D;
            float acc = 0.0f;
            for (int i = 0; i < D; ++i) acc = fmaf(srow[i], rot[grp][i], acc);
            if (valid) a.qproj[(int64_t)head * m + j] = acc * ps;
        }
    }
}

// ----------------------------------------------------------------- split ----
// K side on matrix cores.  For one wave and 16 tokens, the scores of the 16
// query-head columns (G used) are D[token][head] = sum_dim C[token][dim] Q[dim][head]
// with v_mfma_f32_16x16x32_f16: lane l holds A = 8 dims of token l%16 and
// B = the same 8 dims of head l%16, for dims (l/16)*d/4 + 8*ks + [0, 8) in K
// step ks (each lane group owns a contiguous quarter of the dims, so its code
// bytes are one contiguous load).  Float32 accuracy comes from splitting both
// operands into half hi + lo parts: q_hi c_hi + q_lo c_hi + q_hi c_lo (the
// c_lo q_lo term is below float32 rounding).  The query is scaled per head by a
// power of two into [2^14, 2^15) and the centroids by 16 so every lo part is a
// normal half; the scale is removed exactly on the float32 result.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int D, int KB, int VB, int G>
struct Cfg {
    // K side: scores on matrix cores (see above)
    static constexpr int RBK = D * KB / 8;          // K code bytes per token
    static constexpr int CPT = RBK / 16;            // 16-byte chunks per K row
    static constexpr int RBKP = RBK % 64 == 0 ? RBK + 16 : RBK;  // LDS K row stride (bank spread)
    static constexpr int DG = D / 4;                // dims per lane group
    static constexpr int KSTEPS = DG / 8;           // MFMA K steps (32 dims each)
    static constexpr int GB = DG * KB / 8;          // K code bytes per lane group per token
    static constexpr int KLU = (KB == 3) ? 6 : 8;   // bits per K table lookup
    static constexpr int KCPL = KLU / KB;           // codes per lookup
    static constexpr int LPS = 8 / KCPL;            // lookups per K step
    static constexpr int KENT = 4 * KCPL;           // bytes per K table entry: hi[KCPL], lo[KCPL] halves
    static constexpr int KTABB = (1 << KLU) * KENT;
    // V side: weighted sums on matrix cores.  Output column n' of N-block nb is
    // dim NB*n' + nb, so a lane's codes for all N-blocks are one contiguous
    // PIECE-bit field of the token's row.
    static constexpr int RBV = D * VB / 8;          // V code bytes per token
    static constexpr int VTW = RBV / 4;             // dwords per V row
    static constexpr int NB = D / 16;               // N-blocks of 16 columns
    static constexpr int PIECE = VB * NB;           // bits per lane per token
    static constexpr int PL = VB <= 2 ? 2 : 1;      // N-blocks per V table lookup
    static constexpr int VIDXB = 2 * PL * VB;       // V table index bits (two tokens x PL codes)
    static constexpr int VENT = 4 * PL;             // bytes per V table entry (PL half2)
    static constexpr int VTABB = (1 << VIDXB) * VENT;
    // per wave: K tile [64][RBKP] bytes, V tile dword-major [VTW + 1][64],
    // head factors [16], K norm / V norm / gamma [64] floats each
    static constexpr int KT_DW = 64 * RBKP / 4;
    static constexpr int WAVE_DW = KT_DW + (VTW + 1) * 64 + 16 + 3 * 64;
    static constexpr int MAIN = 4 * WAVE_DW;
    static constexpr int MERGE = 4 * G * (D + 2);
    static constexpr int UNION = MAIN > MERGE ? MAIN : MERGE;
};

__device__ __forceinline__ half8_t as_half8(uint4 u) { return __builtin_bit_cast(half8_t, u); }

template <int BITS>
__device__ __forceinline__ uint32_t field_at(const uint32_t* w, int bit0) {
    // bits [bit0, bit0 + BITS) of the little-endian word array (bit0 compile-time after unrolling)
    const int wi = bit0 >> 5, sh = bit0 & 31;
    if (sh + BITS <= 32) return (w[wi] >> sh) & ((1u << BITS) - 1u);
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << BITS) - 1u);
}

// Power of two mapping max|v| of a head (its four lane groups) into [2^14, 2^15).
__device__ __forceinline__ float head_scale(float local_absmax) {
    float mx = fmaxf(local_absmax, xor_lane<16>(local_absmax));
    mx = fmaxf(mx, xor_lane<32>(mx));
    if (!(mx > 0.0f) || !isfinite(mx)) return 1.0f;
    int e;
    frexpf(mx, &e);
    return ldexpf(1.0f, 15 - e);
}

__device__ __forceinline__ float bcast_lane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Loads of one 64-token tile into registers: the K tile as 16-byte chunks
// (chunk 64*j + lane of the tile), the V row of token t0 + lane and its norms.
// Token indices are clamped into [t0, t_end) so every address is valid; values
// of clamped tokens are masked by the caller.
template <int D, int KB, int VB, bool QJL>
__device__ __forceinline__ void fetch_tile(uint32_t (&rk)[D * KB / 32], uint32_t (&rv)[D * VB / 32], uint32_t& rn,
                                           uint32_t& rg, const AttnArgs& a, const uint8_t* kcodes,
                                           const uint8_t* vcodes, int64_t kvrow, int64_t t0, int64_t t_end,
                                           int lane) {
    constexpr int RBK = D * KB / 8, RBV = D * VB / 8, CPT = RBK / 16;
    // token indices fit 32 bits (ctx_cap * row bytes < 2^31 is checked on the host)
    const uint32_t last = (uint32_t)(t_end - 1), tb = (uint32_t)t0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t c = 64 * j + lane;
        uint32_t t = tb + c / CPT;
        t = t < last ? t : last;
        const uint4 v = *reinterpret_cast<const uint4*>(kcodes + (t * RBK + (c % CPT) * 16));
        rk[4 * j] = v.x; rk[4 * j + 1] = v.y; rk[4 * j + 2] = v.z; rk[4 * j + 3] = v.w;
    }
    uint32_t tl = tb + lane;
    tl = tl < last ? tl : last;
    const uint4* vp = reinterpret_cast<const uint4*>(vcodes + tl * RBV);
#pragma unroll
    for (int w = 0; w < RBV / 16; ++w) {
        const uint4 v = vp[w];
        rv[4 * w] = v.x; rv[4 * w + 1] = v.y; rv[4 * w + 2] = v.z; rv[4 * w + 3] = v.w;
    }
    const uint16_t* kn = a.k_norms + kvrow;
    const uint16_t* vn = a.v_norms + kvrow;
    rn = (uint32_t)kn[tl] | ((uint32_t)vn[tl] << 16);
    if constexpr (QJL) rg = (a.k_gamma + kvrow)[tl];
}

template <int D, int KB, int VB, int G, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TQ_SPLIT_WAVES(D)))) void split_kernel(AttnArgs a) {
    using C = Cfg<D, KB, VB, G>;
    constexpr int QJLB = QJL ? 8 * 64 * 8 : 0;   // dwords: QJL B operands (<= 8 K steps x 64 lanes x hi,lo)
    constexpr int SIGB = QJL ? 256 * 4 : 0;      // dwords: sign table 256 x 8 halves
    constexpr int SMEM = C::KTABB / 4 + C::VTABB / 4 + C::UNION + QJLB + SIGB;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SMEM];
    uint8_t* ktab = reinterpret_cast<uint8_t*>(smem);
    uint8_t* vtab = reinterpret_cast<uint8_t*>(smem + C::KTABB / 4);
    uint32_t* uni = smem + C::KTABB / 4 + C::VTABB / 4;
    uint4* qjlb = reinterpret_cast<uint4*>(uni + C::UNION);
    uint4* sigt = reinterpret_cast<uint4*>(uni + C::UNION + QJLB);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.chunks, chunk = blockIdx.y - kvh * a.chunks;
    const int b = blockIdx.z;
    const int m = QJL ? a.kc.qjl_m : 0;
    int64_t ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
    const int64_t t_beg = (int64_t)split * a.split_tokens;
    const int64_t t_end = (t_beg + a.split_tokens < ctx) ? t_beg + a.split_tokens : ctx;
    const int h0 = kvh * a.g + chunk * G;

    // K table: entry u -> 16*c_K of its KCPL codes, half hi parts then lo parts
    for (int u = tid; u < (1 << C::KLU); u += 256) {
        _Float16* e = reinterpret_cast<_Float16*>(ktab + u * C::KENT);
#pragma unroll
        for (int p = 0; p < C::KCPL; ++p) {
            const float c = 16.0f * a.kc.centroid[(u >> (KB * p)) & ((1 << KB) - 1)];
            const _Float16 hi = (_Float16)c;
            e[p] = hi;
            e[C::KCPL + p] = (_Float16)(c - (float)hi);
        }
    }
    // V table: index = (PL codes of token a) | (PL codes of token b) << PL*VB;
    // entry dword q = half2(c_V[code_q of a], c_V[code_q of b])
    for (int u = tid; u < (1 << C::VIDXB); u += 256) {
        _Float16* e = reinterpret_cast<_Float16*>(vtab + u * C::VENT);
        constexpr int VM = (1 << VB) - 1;
#pragma unroll
        for (int q = 0; q < C::PL; ++q) {
            e[2 * q] = (_Float16)a.vc.centroid[(u >> (q * VB)) & VM];
            e[2 * q + 1] = (_Float16)a.vc.centroid[(u >> (C::PL * VB + q * VB)) & VM];
        }
    }
    if constexpr (QJL) {
        _Float16* st = reinterpret_cast<_Float16*>(sigt);
        for (int e = tid; e < 256 * 8; e += 256) st[e] = ((e >> 3) >> (e & 7)) & 1 ? (_Float16)1.0f : (_Float16)(-1.0f);
    }

    // K-side B operands: rotated query (and QJL projection) of head n, scaled
    // by one power of two per head; zero for n >= G
    const float* qrot = a.qrot + ((int64_t)b * a.hq + h0) * D;  // [dim][G] inside this chunk
    half8_t qhi[C::KSTEPS], qlo[C::KSTEPS];
    float qinv;
    {
        float qv[C::KSTEPS][8];
        float amax = 0.0f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int dim = grp * C::DG + 8 * ks + j;
                qv[ks][j] = n < G ? qrot[dim * G + n] : 0.0f;
                amax = fmaxf(amax, fabsf(qv[ks][j]));
            }
        const float* qp = a.qproj + ((int64_t)b * a.hq + h0) * m;
        if constexpr (QJL) {
            for (int ks = 0; ks < (m >> 5); ++ks)
                for (int j = 0; j < 8; ++j)
                    amax = fmaxf(amax, n < G ? fabsf(qp[n * m + grp * (m >> 2) + 8 * ks + j]) : 0.0f);
        }
        const float sc = head_scale(amax);
        qinv = 1.0f / (16.0f * sc);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = qv[ks][j] * sc;
                const _Float16 hi = (_Float16)v;
                qhi[ks][j] = hi;
                qlo[ks][j] = (_Float16)(v - (float)hi);
            }
        if constexpr (QJL) {
            if (wave == 0) {
                for (int ks = 0; ks < (m >> 5); ++ks) {
                    half8_t hi8, lo8;
                    for (int j = 0; j < 8; ++j) {
                        // the sign operand carries 16*gamma, so scale by sc only
                        const float v = (n < G ? qp[n * m + grp * (m >> 2) + 8 * ks + j] : 0.0f) * sc;
                        const _Float16 hi = (_Float16)v;
                        hi8[j] = hi;
                        lo8[j] = (_Float16)(v - (float)hi);
                    }
                    qjlb[(ks * 64 + lane) * 2] = __builtin_bit_cast(uint4, hi8);
                    qjlb[(ks * 64 + lane) * 2 + 1] = __builtin_bit_cast(uint4, lo8);
                }
            }
        }
    }
    __syncthreads();

    const int64_t kvrow = ((int64_t)b * a.hkv + kvh) * a.ctx_cap;
    const uint8_t* kcodes = a.k_codes + kvrow * C::RBK;
    const uint8_t* vcodes = a.v_codes + kvrow * (C::RBV);
    uint32_t* wv = uni + wave * C::WAVE_DW;
    uint8_t* kt = reinterpret_cast<uint8_t*>(wv);       // [64][RBKP] K tile
    uint32_t* vt = wv + C::KT_DW;                       // [VTW + 1][64] dword-major V tile
    float* hfac = reinterpret_cast<float*>(vt + (C::VTW + 1) * 64);  // [16] per-head V factors
    float* knl = hfac + 16;                             // [64] K norms
    float* vnl = knl + 64;                              // [64] V norms * weight scale
    float* gml = vnl + 64;                              // [64] QJL gamma

    float m_run = -INFINITY, l_lane = 0.0f;  // head n's running max / this lane's partial sum
    // V sums D[nb][i]: head 4*grp + i, dim NB*n + nb, in units of the current weight scale
    floatx4_t vacc[C::NB];
#pragma unroll
    for (int q = 0; q < C::NB; ++q) vacc[q] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    int wexp_prev = 0;
    bool first = true;
    constexpr int PB0 = 0;
    const int pbit = C::PIECE * n;               // this lane's V field inside a row
    const int pw0 = pbit >> 5, psh = pbit & 31;  // first dword and shift
    (void)PB0;

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int64_t t0 = t_beg + wave_u * 64;
    uint32_t rk[4 * C::CPT];
    uint32_t rv[C::VTW], rn = 0, rg = 0;
    if (t0 < t_end) fetch_tile<D, KB, VB, QJL>(rk, rv, rn, rg, a, kcodes, vcodes, kvrow, t0, t_end, lane);
    for (; t0 < t_end; t0 += 256) {
        const int rem = (int)(t_end - t0);  // tokens left in this split (> 0)
        const bool lane_valid = lane < rem;
        // ---- stage this tile: K chunks (row-major, padded rows), V (dword-major), norms
#pragma unroll
        for (int j = 0; j < C::CPT; ++j) {
            const int c = 64 * j + lane;
            *reinterpret_cast<uint4*>(kt + (c / C::CPT) * C::RBKP + (c % C::CPT) * 16) =
                make_uint4(rk[4 * j], rk[4 * j + 1], rk[4 * j + 2], rk[4 * j + 3]);
        }
#pragma unroll
        for (int w = 0; w < C::VTW; ++w) vt[w * 64 + lane] = rv[w];
        vt[C::VTW * 64 + lane] = 0u;
        const float vnf = lane_valid ? half_bits_to_float(rn >> 16) : 0.0f;
        knl[lane] = lane_valid ? half_bits_to_float(rn & 0xFFFFu) : 0.0f;
        if constexpr (QJL) gml[lane] = half_bits_to_float(rg);
        // power of two bringing this tile's largest V norm into [2^14, 2^15)
        float vmax = vnf;
        vmax = fmaxf(vmax, xor_lane<1>(vmax));
        vmax = fmaxf(vmax, xor_lane<2>(vmax));
        vmax = fmaxf(vmax, xor_lane<4>(vmax));
        vmax = fmaxf(vmax, xor_lane<8>(vmax));
        vmax = fmaxf(vmax, xor_lane<16>(vmax));
        vmax = fmaxf(vmax, xor_lane<32>(vmax));
        int wexp = 0;
        if (vmax > 0.0f && isfinite(vmax)) frexpf(vmax, &wexp);
        vnl[lane] = vnf * ldexpf(1.0f, 15 - wexp);  // weights are p * vn * 2^(15 - wexp)
        // ---- fetch the next tile while this one computes (clamped: always valid)
        fetch_tile<D, KB, VB, QJL>(rk, rv, rn, rg, a, kcodes, vcodes, kvrow, t0 + 256, t_end, lane);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- K scores on matrix cores: 4 sub-tiles of 16 tokens
        floatx4_t sacc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t kg[C::GB / 4];
            const uint8_t* src = kt + (16 * j + n) * C::RBKP + grp * C::GB;
            if constexpr (C::GB % 16 == 0) {
#pragma unroll
                for (int w = 0; w < C::GB / 16; ++w) {
                    const uint4 v = reinterpret_cast<const uint4*>(src)[w];
                    kg[4 * w] = v.x; kg[4 * w + 1] = v.y; kg[4 * w + 2] = v.z; kg[4 * w + 3] = v.w;
                }
            } else if constexpr (C::GB % 8 == 0) {
#pragma unroll
                for (int w = 0; w < C::GB / 8; ++w) {
                    const uint2 v = reinterpret_cast<const uint2*>(src)[w];
                    kg[2 * w] = v.x; kg[2 * w + 1] = v.y;
                }
            } else {
#pragma unroll
                for (int w = 0; w < C::GB / 4; ++w) kg[w] = reinterpret_cast<const uint32_t*>(src)[w];
            }
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int u = 0; u < C::LPS; ++u) {
                    const uint32_t f = field_at<C::KLU>(kg, ks * 8 * KB + u * C::KLU);
                    const uint8_t* ent = ktab + f * C::KENT;
                    if constexpr (C::KCPL == 2) {
                        const uint2 e = *reinterpret_cast<const uint2*>(ent);
                        hw[u] = e.x;
                        lw[u] = e.y;
                    } else if constexpr (C::KCPL == 4) {
                        const uint4 e = *reinterpret_cast<const uint4*>(ent);
                        hw[2 * u] = e.x; hw[2 * u + 1] = e.y;
                        lw[2 * u] = e.z; lw[2 * u + 1] = e.w;
                    } else {
                        const uint4 eh = reinterpret_cast<const uint4*>(ent)[0];
                        const uint4 el = reinterpret_cast<const uint4*>(ent)[1];
                        hw[0] = eh.x; hw[1] = eh.y; hw[2] = eh.z; hw[3] = eh.w;
                        lw[0] = el.x; lw[1] = el.y; lw[2] = el.z; lw[3] = el.w;
                    }
                }
                const half8_t ahi = as_half8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
                const half8_t alo = as_half8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, qhi[ks], sacc[j], 0, 0, 0);
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, qlo[ks], sacc[j], 0, 0, 0);
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, qhi[ks], sacc[j], 0, 0, 0);
            }
        }
        if constexpr (QJL) {
            // A = 16*gamma*(+-1) of token 16j + n (exact in half); same accumulators
            const int gbytes = m >> 5;
            for (int j = 0; j < 4; ++j) {
                int64_t t = t0 + 16 * j + n;
                t = t < t_end - 1 ? t : t_end - 1;
                const _Float16 g16 = (_Float16)(16.0f * gml[16 * j + n]);
                const uint8_t* sp = a.k_qjl + (kvrow + t) * (m >> 3) + grp * gbytes;
                for (int ks = 0; ks < (m >> 5); ++ks) {
                    const half8_t asg = as_half8(sigt[sp[ks]]) * g16;
                    sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(asg, as_half8(qjlb[(ks * 64 + lane) * 2]), sacc[j], 0, 0, 0);
                    sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(asg, as_half8(qjlb[(ks * 64 + lane) * 2 + 1]), sacc[j], 0, 0, 0);
                }
            }
        }
        // ---- scores of tokens 16j + 4*grp + v for head n; online softmax (log2 domain)
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 kn4 = *reinterpret_cast<const float4*>(knl + 16 * j + 4 * grp);
            const float knv[4] = {kn4.x, kn4.y, kn4.z, kn4.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool ok = 16 * j + 4 * grp + v < rem;
                const float sv = ok ? sacc[j][v] * qinv * knv[v] : -INFINITY;
                sacc[j][v] = sv;
                tmax = fmaxf(tmax, sv);
            }
        }
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        const float mnew = fmaxf(m_run, tmax);
        const float alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
        // V-side A operands: half weights of this lane's tokens (K order: sub-tile
        // pairs (2s, 2s+1), tokens 4*grp + v), head n = row
        uint32_t wa[2][4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 vn4 = *reinterpret_cast<const float4*>(vnl + 16 * j + 4 * grp);
            const float p0 = fast_exp2(sacc[j][0] - mnew), p1 = fast_exp2(sacc[j][1] - mnew);
            const float p2 = fast_exp2(sacc[j][2] - mnew), p3 = fast_exp2(sacc[j][3] - mnew);
            psum += (p0 + p1) + (p2 + p3);
            wa[j >> 1][2 * (j & 1)] = pack_half2(p0 * vn4.x, p1 * vn4.y);
            wa[j >> 1][2 * (j & 1) + 1] = pack_half2(p2 * vn4.z, p3 * vn4.w);
        }
        l_lane = fmaf(l_lane, alpha, psum);
        // per-head factor for the V sums: softmax correction x change of weight scale
        const float rescale = first ? 1.0f : ldexpf(1.0f, wexp_prev - wexp);  // exact power of two
        wexp_prev = wexp;
        first = false;
        if (grp == 0) hfac[n] = alpha * rescale;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            const float4 f4 = *reinterpret_cast<const float4*>(hfac + 4 * grp);
#pragma unroll
            for (int q = 0; q < C::NB; ++q) {
                vacc[q][0] *= f4.x;
                vacc[q][1] *= f4.y;
                vacc[q][2] *= f4.z;
                vacc[q][3] *= f4.w;
            }
        }

        // ---- V sums on matrix cores: for K step s (sub-tiles 2s, 2s+1), this
        // lane's 8 tokens, its PIECE-bit field of each token's V row
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t pc[8];  // PIECE <= 32: the field; else its low 32 bits (high part in ph)
            uint32_t ph[8];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int tok = 16 * (2 * s2 + jj) + 4 * grp;
                const uint4 x = *reinterpret_cast<const uint4*>(vt + pw0 * 64 + tok);
                uint32_t lo[4] = {x.x, x.y, x.z, x.w};
                if constexpr (C::PIECE <= 32 && (32 % C::PIECE == 0)) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) pc[4 * jj + v] = lo[v] >> psh;
                } else {
                    const uint4 y = *reinterpret_cast<const uint4*>(vt + (pw0 + 1) * 64 + tok);
                    const uint32_t hi[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        pc[4 * jj + v] = __builtin_amdgcn_alignbit(hi[v], lo[v], psh);
                        ph[4 * jj + v] = psh == 0 ? hi[v] : (hi[v] >> psh);
                    }
                }
            }
            const half8_t aw = as_half8(make_uint4(wa[s2][0], wa[s2][1], wa[s2][2], wa[s2][3]));
#pragma unroll
            for (int k = 0; k < C::NB / C::PL; ++k) {
                constexpr int FB = C::PL * VB;  // bits per token per lookup
                uint32_t bw[C::PL][4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const int bit = k * FB;
                    uint32_t fa, fb;
                    if constexpr (C::PIECE <= 32) {
                        fa = (pc[2 * pp] >> bit) & ((1u << FB) - 1u);
                        fb = (pc[2 * pp + 1] >> bit) & ((1u << FB) - 1u);
                    } else {
                        const uint64_t xa = ((uint64_t)ph[2 * pp] << 32) | pc[2 * pp];
                        const uint64_t xb = ((uint64_t)ph[2 * pp + 1] << 32) | pc[2 * pp + 1];
                        fa = (uint32_t)(xa >> bit) & ((1u << FB) - 1u);
                        fb = (uint32_t)(xb >> bit) & ((1u << FB) - 1u);
                    }
                    const uint32_t idx = fa | (fb << FB);
                    if constexpr (C::PL == 2) {
                        const uint2 e = *reinterpret_cast<const uint2*>(vtab + idx * 8);
                        bw[0][pp] = e.x;
                        bw[1][pp] = e.y;
                    } else {
                        bw[0][pp] = *reinterpret_cast<const uint32_t*>(vtab + idx * 4);
                    }
                }
#pragma unroll
                for (int q = 0; q < C::PL; ++q) {
                    const half8_t bv = as_half8(make_uint4(bw[q][0], bw[q][1], bw[q][2], bw[q][3]));
                    vacc[k * C::PL + q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bv, vacc[k * C::PL + q], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // block merge of the four waves (V sums back to true units)
    const float wunit = ldexpf(1.0f, wexp_prev - 15);
    float l_head = l_lane + xor_lane<16>(l_lane);
    l_head += xor_lane<32>(l_head);
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(uni);  // [4][G][D + 2]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float mh = bcast_lane(m_run, h);
        const float lh = bcast_lane(l_head, h);
        if (lane == 0) {
            mrg[(wave * G + h) * (D + 2)] = mh;
            mrg[(wave * G + h) * (D + 2) + 1] = lh;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * grp + i;
        if (h < G) {
            float* rr = mrg + (wave * G + h) * (D + 2) + 2 + C::NB * n;
#pragma unroll
            for (int q = 0; q < C::NB; ++q) rr[q] = vacc[q][i] * wunit;
        }
    }
    __syncthreads();
    float* part = a.part + (((int64_t)b * a.hq + h0) * a.splits + split) * (D + 2);
    const int64_t hstride = (int64_t)a.splits * (D + 2);
    for (int e = tid; e < G * (D + 2); e += 256) {
        const int h = e / (D + 2), i = e - h * (D + 2);
        float mw[4], mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = mrg[(w * G + h) * (D + 2)];
            mx = fmaxf(mx, mw[w]);
        }
        float val;
        if (i == 0) {
            val = mx;
        } else if (mx == -INFINITY) {
            val = 0.0f;
        } else {
            val = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) val = fmaf(mrg[(w * G + h) * (D + 2) + i], exp2f(mw[w] - mx), val);
        }
        part[h * hstride + i] = val;
    }
}

// --------------------------------------------------------------- combine ----
// One block of 256 threads per (batch, query head): 256/D split groups reduce
// disjoint subsets of the splits with independent (unrolled) loads, the
// groups are merged through LDS, then one inverse transform.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
    constexpr int NG = 256 / D;  // split groups
    __shared__ float x[NG][D];
    __shared__ float red[256];
    __shared__ float lsum[NG];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int i = tid % D, grp = tid / D;
    const float* p = a.part + (int64_t)bh * a.splits * (D + 2);
    const int S = a.splits;

    float mx = -INFINITY;
    for (int s = tid; s < S; s += 256) mx = fmaxf(mx, p[(int64_t)s * (D + 2)]);
    red[tid] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    mx = red[0];
    float L = 0.0f, acc = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll 8
        for (int s = grp; s < S; s += NG) {
            const float* ps = p + (int64_t)s * (D + 2);
            const float f = exp2f(ps[0] - mx);
            L = fmaf(ps[1], f, L);
            acc = fmaf(ps[2 + i], f, acc);
        }
    }
    x[grp][i] = acc;
    if (i == 0) lsum[grp] = L;
    __syncthreads();
    if (grp == 0) {
        float at = 0.0f, lt = 0.0f;
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) {
            at += x[g2][i];
            lt += lsum[g2];
        }
        x[0][i] = lt > 0.0f ? at / lt : 0.0f;
    }
    __syncthreads();
    // inverse rotation: D_V H(x) / d
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
        float nv = 0.0f;
        if (grp == 0) nv = ((i & h) == 0) ? x[0][i] + x[0][i + h] : x[0][i - h] - x[0][i];
        __syncthreads();
        if (grp == 0) x[0][i] = nv;
        __syncthreads();
    }
    if (grp == 0) {
        const uint32_t neg = ((a.vc.sign_mask[i >> 5] >> (i & 31)) & 1u) << 31;
        a.out[(int64_t)bh * D + i] = as_f(as_u(x[0][i] * (1.0f / (float)D)) ^ neg);
    }
}

template <int D, int KB, int VB, int G>
hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
    dim3 grid(a.splits, a.hkv * a.chunks, a.batch);
    if (a.kc.qjl_m > 0)
        hipLaunchKernelGGL((split_kernel<D, KB, VB, G, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((split_kernel<D, KB, VB, G, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t launch_split_g(const AttnArgs& a, hipStream_t s) {
    switch (a.heads_per_chunk) {
        case 1: return launch_split<D, KB, VB, 1>(a, s);
        case 2: return launch_split<D, KB, VB, 2>(a, s);
        case 3: return launch_split<D, KB, VB, 3>(a, s);
        case 4: return launch_split<D, KB, VB, 4>(a, s);
        case 5: return launch_split<D, KB, VB, 5>(a, s);
        case 6: return launch_split<D, KB, VB, 6>(a, s);
        case 7: return launch_split<D, KB, VB, 7>(a, s);
        default: return launch_split<D, KB, VB, 8>(a, s);
    }
}

template <int D, int KB>
hipError_t launch_split_dk(const AttnArgs& a, hipStream_t s) {
    switch (a.vc.bits) {
        case 1: return launch_split_g<D, KB, 1>(a, s);
        case 2: return launch_split_g<D, KB, 2>(a, s);
        case 3: return launch_split_g<D, KB, 3>(a, s);
        default: return launch_split_g<D, KB, 4>(a, s);
    }
}

}  // namespace attn

// One explicit instantiation per (D, KB) lives in its own translation unit.
template <int D, int KB>
hipError_t launch_split_dk(const AttnArgs& a, hipStream_t s);

}  // namespace tqi
