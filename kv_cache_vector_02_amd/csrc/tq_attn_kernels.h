// Decode attention over the packed cache, gfx950.
//
// Launches per call (two without QJL):
//   1. qprep (QJL keys only): S q_rot / sqrt(d) per query head, with
//      q_rot = H(D_K q) from the register/DPP transform.
//   2. split: grid (splits, kv_head x head_chunk, batch), one block per compute
//      unit.  The block first rotates its chunk's queries (q_rot = H(D_K q),
//      pre-scaled by scale * log2(e) / d).  Each wave then streams 64-token tiles of its split: K scores on the
//      matrix cores from centroid pairs looked up in LDS tables by the K codes
//      (loaded straight into the operand layout), a wave-wide online softmax in
//      the log2 domain, then the V sums on the matrix cores with the softmax
//      weights as one operand and V centroids looked up by the V codes (staged
//      through LDS) as the other, accumulated in the rotated domain.  The waves
//      of a block merge their (max, sum, acc) and write one partial.
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


// Score factor alpha(N) of a query row that attends over n tokens (1 when the
// mode is plain or n <= 1): the dynamic sharpening and MMSE softening of the
// llama.cpp fork's README ("TurboQuant KV 캐시 압축 for llama.cpp", v1.5.2
// "Attention Sharpening — 이론 & 동적 α 공식" and "핵심 변경" item 11).
__device__ __forceinline__ float score_factor(const AttnArgs& a, int n) {
    if (a.score_mode == 0 || n <= 1) return 1.0f;
    const float ln_n = logf((float)n);
    if (a.score_mode == 1) return 1.0f + a.sharp_c * sqrtf(ln_n);
    return a.sqnr / (a.sqnr + sqrtf(ln_n * a.inv_ln_n0));
}

// Tokens query row `row` ((b * ncols + c) * hq + h) attends over.
__device__ __forceinline__ int row_tokens(const AttnArgs& a, int64_t row) {
    const int64_t bc = row / a.hq;
    const int b = (int)(bc / a.ncols), c = (int)(bc - (int64_t)b * a.ncols);
    const int cap = (int)a.ctx_cap;
    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int n = ctx - (a.ncols - 1 - c);
    return n > 0 ? n : 0;
}

// ----------------------------------------------------------------- qprep ----
// Keys with residual bits only: per query row, the projection S H(D_K q) /
// sqrt(d) of the rotated query (the Q_wht2 side of the fused query pass),
// pre-scaled by scale * log2(e) * sqrt(pi/2) / m (S = H D2 for the SRHT kind;
// S = I and the constant 1 for Direct Sign).  The scan rotates its queries
// itself.
template <int D, int DT>
__global__ __launch_bounds__(64) void qprep_kernel(AttnArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    __shared__ float rot[VPW][D];
    const int lane = threadIdx.x;
    const int gl = lane & (LPV - 1), grp = lane / LPV;
    const int heads = a.batch * a.ncols * a.hq;
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
    if constexpr (D == 64) {
        if (a.kc.rotation == TQ_ROT_DOUBLE) second_pass<LPV>(v, gl, a.kc.sign_mask3);
    }
    const int m = a.kc.qjl_m;
    const float alpha = valid ? score_factor(a, row_tokens(a, head)) : 1.0f;
    if (a.kc.residual != TQ_RES_QJL) {
        // m = D: the structured SRHT projection H(D2 q_rot) (second sign flip
        // and transform in registers), or Direct Sign's q_rot itself with the
        // constant 1 in place of sqrt(pi/2)/m
        float ps = a.scale * kLog2e / sqrtf((float)D) * alpha;
        if (a.kc.residual == TQ_RES_SRHT) {
            const uint32_t sbits2 = (a.kc.sign_mask2[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e]) ^ (((sbits2 >> e) & 1u) << 31));
            fwht<LPV>(v, gl);
            ps *= sqrtf(1.57079632679489662f) / (float)m;
        }
        if (valid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a.qproj[(int64_t)head * m + gl * 8 + e] = v[e] * ps;
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rot[grp][gl * 8 + e] = v[e];
    __syncthreads();
    const float ps = a.scale * kLog2e * sqrtf(1.57079632679489662f) / ((float)m * sqrtf((float)D)) * alpha;
    for (int j = gl; j < m; j += LPV) {
        const float* srow = a.S + (int64_t)j * D;
        float acc = 0.0f;
        for (int i = 0; i < D; ++i) acc = fmaf(srow[i], rot[grp][i], acc);
        if (valid) a.qproj[(int64_t)head * m + j] = acc * ps;
    }
}

// ----------------------------------------------------------------- split ----
// Both contractions of a 64-token tile run on v_mfma_f32_16x16x32_f16.  For
// this MFMA lane l holds A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16]
// (e = 0..7) and receives D[4(l/16) + i][l%16] (i = 0..3).
//
// Scores, per 16-token sub-tile j: D[token][col] = sum_k A[token][k] B[k][col].
// Lane (n, grp) = (l%16, l/16) takes the K codes of token 16j + n straight from
// memory, dims grp*d/4 + [0, d/4) (one contiguous load); K step ks covers dims
// grp*d/4 + 4ks + [0, 4).  Float32 accuracy comes from splitting both operands
// into half hi + lo parts, folded into the two MFMA dimensions that have room:
// the eight k slots of a lane hold c_hi and c_lo of its four dims, and columns
// 0..7 hold q_hi of the (at most eight) query heads while columns 8..15 hold
// q_lo, so that D[t][h] + D[t][h + 8] = sum_dim (c_hi + c_lo)(q_hi + q_lo) over
// the centroid and query of every dim, a float32-exact product up to the
// rounding of the accumulation (the c_lo * q_lo term, below 2^-22 of the
// score, is zeroed out of the q_lo columns).  The query chunk is scaled by one power of two
// into [2^14, 2^15) and the centroids by 16 so every lo part is a normal half;
// the scale is removed exactly on the float32 result.  After adding the two
// column halves (a DPP row rotate), lane (n, grp) holds the scores of tokens
// 16j + 4grp + i for head n % 8.
//
// V sums, per K step s2 of 32 tokens: D[head][col] = sum_token W[head][token]
// C_V[token][dim(col)], with the softmax weights of the lane's own registers as
// A (k slot 8grp + e <-> token 32 s2 + 16(e/4) + 4grp + e%4) and column n' of
// N-block nb standing for dim NB*n' + nb, so a lane's codes of one token are one
// contiguous NB*VB-bit piece of the token's row.  Centroids come from an LDS
// table indexed by VT codes of one token; v_perm pairs the halves of two tokens
// into one B dword.  Rows 8..15 repeat heads 0..7 and are not used.
//
// Softmax: the log2-domain scores are exponentiated against a reference max
// that is only raised when a score exceeds it by more than 2^kTauLog2 (lazy
// rescaling), and the V weights p * |v| are scaled by a power of two taken
// from a reference V norm that is only raised when a larger norm shows up.
// Both keep the half weights below 2^15; the rare raise rescales the running
// sums of the wave.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr float kTauLog2 = 12.0f;  // scores may exceed the reference max by this much (log2 units)
constexpr int kVHeadroom = 1;     // binades of headroom above the largest V norm seen
constexpr int kKLookahead = 2;    // K table lookups issued this many matrix-core steps ahead

// LDS of one split block: the lookup tables, one staging area per wave and,
// with QJL, the sign-side operands.  gfx950 reads 256 bytes per clock from 64
// four-byte banks (32 lanes per pass for 8-byte reads, 16 for 16-byte reads).
//
// Split tables: a K table and a V table of 256-byte rows, row u holding the
// entry of index u repeated across the whole row (256 / entry-size slices).
// Lane l reads slice l % slices, so the lanes of one pass touch distinct banks
// whatever their indices.  When the two tables and the wave areas do not fit,
// one shared table of 256-byte rows holds the K entry in its first and the V
// entry in its last 128 bytes (half the slices: two lanes of a pass may share a
// bank).  Either way a row offset is index * 256 (one byte permute of an 8-bit
// index).
constexpr int kLdsBytes = 160 * 1024;
constexpr int kVStride = 68;                        // padded dword stride of the V staging rows
constexpr int k_codes(int kb) { return kb >= 3 ? 2 : 4; }  // codes per K lookup
constexpr int v_codes(int vb) { return vb == 1 ? 8 : (vb == 2 ? 4 : 2); }  // codes per V lookup
constexpr int wave_dw(int d, int vb) { return (d * vb / 32 + 1) * kVStride + 16 + 3 * 64 + (d == 256 ? 2 * 64 : 0); }
constexpr int qjl_dw(bool qjl) { return qjl ? 8 * 64 * 4 + 256 * 4 : 0; }
constexpr int k_rows(int kb) { return 1 << (k_codes(kb) * kb); }
constexpr int v_rows(int vb) { return 1 << (v_codes(vb) * vb); }
constexpr int split_tab_bytes(int kb, int vb) { return (k_rows(kb) + v_rows(vb)) * 256; }
constexpr int shared_tab_bytes(int kb, int vb) { return (k_rows(kb) > v_rows(vb) ? k_rows(kb) : v_rows(vb)) * 256; }
constexpr bool split_fits(int d, int kb, int vb, bool qjl, int nw) {
    return split_tab_bytes(kb, vb) + 4 * (nw * wave_dw(d, vb) + qjl_dw(qjl)) <= kLdsBytes;
}
// Waves of one split block (the block owns a compute unit: one resident block
// per CU, its waves sharing the tables): 8 up to d = 128 (two waves per SIMD,
// 256 registers each), 4 at d = 256 (one wave per SIMD: the twice longer query
// operands and V sums need up to 512 registers).  No variant then spills in
// its tile loop; with 12 waves (168 registers) most d = 128 variants
// spilled and ran up to 1.7x slower, with 8 waves at d = 256 up to 2.3x.  The
// split tables are used where they fit beside the wave areas, else the shared
// table; the QJL variant, whose extra operands take LDS, keeps the shared one.
constexpr int split_waves(int d, int kb, int vb, bool qjl) {
    (void)kb, (void)vb, (void)qjl;
    return d >= 256 ? 4 : 8;
}
constexpr bool split_tables(int d, int kb, int vb, bool qjl) {
    return !qjl && split_fits(d, kb, vb, qjl, split_waves(d, kb, vb, qjl));
}
// Blocks of up to 16 query rows (see split_kernel): without QJL and up to
// d = 128, where the 16 rotated query rows fit the wave areas.
constexpr bool split_rows16(int d, bool qjl) { return !qjl && d <= 128; }

template <int D, int KB, int VB, bool QJL, bool TWO = false>
struct Cfg {
    static_assert(!TWO || (D == 256 && !QJL), "the per-half layout is for d = 256 without QJL");
    static constexpr int GMAX = split_rows16(D, QJL) ? 16 : 8;  // query rows per block (at most)
    static constexpr int NW = split_waves(D, KB, VB, QJL);  // waves per block
    static constexpr int NT = 64 * NW;              // threads per block
    // K side
    static constexpr int RBK = D * KB / 8;          // K code bytes per token
    static constexpr int DG = D / 4;                // dims per lane group
    static constexpr int KSTEPS = DG / 4;           // MFMA K steps (4 dims per lane each)
    static constexpr int GB = DG * KB / 8;          // K code bytes per lane group per token
    static constexpr int GW = GB / 4;               // ... in dwords
    static constexpr int KE = k_codes(KB);          // codes per K lookup
    static constexpr int KLU = KE * KB;             // K index bits
    static constexpr int KENT = 4 * KE;             // bytes per K entry: hi halves then lo halves
    static constexpr int LPS = 4 / KE;              // K lookups per step
    // V side
    static constexpr int RBV = D * VB / 8;          // V code bytes per token
    static constexpr int VTW = RBV / 4;             // dwords per V row
    static constexpr int NB = D / 16;               // N-blocks of 16 columns
    static constexpr int PIECE = VB * NB;           // bits per lane per token
    static constexpr int VT = v_codes(VB);          // codes per V lookup
    static constexpr int VLB = VT * VB;             // V index bits
    static constexpr int VENT = 2 * VT;             // bytes per V entry
    static constexpr int VENTW = VENT / 4;          // ... in dwords
    static constexpr int VLK = NB / VT;             // V lookups per token
    // caches with two norm blocks (d = 256): every K step and every V sum
    // covers dims of one half of the rotated vector only (see fetch_k and the V
    // pieces), so a norm per half can scale each half's products
    static constexpr bool HALVES = TWO;
    // tables (see above): slices per row, table bytes, byte offset of V row 0
    // split into the part above 64 KiB (carried by the lane offset) and the
    // rest (an instruction offset)
    static constexpr bool SPLIT = split_tables(D, KB, VB, QJL);
    static constexpr int KROWS = k_rows(KB), VROWS = v_rows(VB);
    static constexpr int KSL = (SPLIT ? 256 : 128) / KENT;  // K slices
    static constexpr int VSL = (SPLIT ? 256 : 128) / VENT;  // V slices
    static constexpr int TABB = SPLIT ? split_tab_bytes(KB, VB) : shared_tab_bytes(KB, VB);
    static constexpr int VBASE = SPLIT ? KROWS * 256 : 128;
    static constexpr uint32_t VOFF0 = SPLIT ? (uint32_t)VBASE & ~0xFFFFu : (uint32_t)VBASE;
    static constexpr int VIMM = SPLIT ? VBASE & 0xFFFF : 0;
    // per wave: V tile dword-major [VTW + 1][VSTR] (last row zero; VSTR pads the
    // rows across banks), head factors [16], K norm * query scale [64], scaled
    // V norm [64], QJL gamma [64]
    static constexpr int VSTR = kVStride;
    static constexpr int WAVE_DW = wave_dw(D, VB);
    static constexpr int QJL_DW = qjl_dw(QJL);      // QJL B operands + sign table
    static constexpr int LOOP_DW = TABB / 4 + NW * WAVE_DW + QJL_DW;
    static constexpr int MERGE_DW = NW * GMAX * (D + 2) + GMAX * (NW + 1);  // partials, then merge factors
    static constexpr int SMEM_DW = LOOP_DW > MERGE_DW ? LOOP_DW : MERGE_DW;
    static_assert(4 * SMEM_DW <= kLdsBytes, "split kernel exceeds LDS");
    static_assert(GMAX * D <= NW * WAVE_DW, "rotated queries exceed the wave areas");
    // K codes double-buffered (loaded a whole tile ahead) where the register
    // budget of two waves per SIMD leaves room
    static constexpr bool KDB = NW <= 8 && !QJL;
};

__device__ __forceinline__ half8_t as_half8(uint4 u) { return __builtin_bit_cast(half8_t, u); }

template <int BITS>
__device__ __forceinline__ uint32_t field_at(const uint32_t* w, int bit0) {
    // bits [bit0, bit0 + BITS) of the little-endian word array (bit0 compile-time after unrolling)
    const int wi = bit0 >> 5, sh = bit0 & 31;
    if (sh + BITS <= 32) return (w[wi] >> sh) & ((1u << BITS) - 1u);
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << BITS) - 1u);
}

__device__ __forceinline__ float bcast_lane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, half2_t));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, xor_lane<1>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<16>(v));
    return fmaxf(v, xor_lane<32>(v));
}

template <int N>
__device__ __forceinline__ void lds_read(uint32_t* dst, const uint8_t* p) {
    if constexpr (N == 1) {
        dst[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (N == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        dst[0] = v.x; dst[1] = v.y;
    } else {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
}

// K codes of sub-tiles 0..3 in MFMA A layout: token t0 + 16j + n, bytes grp*GB.
// With HALVES the lane group's dims are [32 grp, 32 grp + 32) of each half:
// the GB/2 bytes at grp*GB/2 and at RBK/2 + grp*GB/2, one after the other in
// the registers (so K step ks < KSTEPS/2 reads the first half's dims).
// Token indices are clamped into [t0, t_end) so every address is valid.
template <class C>
__device__ __forceinline__ void fetch_k(uint32_t (&rk)[4 * C::GW], const uint8_t* kcodes, uint32_t t0, uint32_t last,
                                        int n, int grp) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t t = t0 + 16 * j + n;
        t = t < last ? t : last;
        if constexpr (C::HALVES) {
            constexpr int HW = C::GW / 2;  // dwords per half
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const uint32_t* p = reinterpret_cast<const uint32_t*>(kcodes + (t * C::RBK + hf * (C::RBK / 2) +
                                                                                  grp * (C::GB / 2)));
                uint32_t* r = rk + j * C::GW + hf * HW;
                if constexpr (HW % 4 == 0) {
#pragma unroll
                    for (int w = 0; w < HW / 4; ++w) {
                        const uint4 v = ld_stream4(p + 4 * w);
                        r[4 * w] = v.x; r[4 * w + 1] = v.y; r[4 * w + 2] = v.z; r[4 * w + 3] = v.w;
                    }
                } else if constexpr (HW % 2 == 0) {
#pragma unroll
                    for (int w = 0; w < HW / 2; ++w) {
                        const uint2 v = ld_stream2(p + 2 * w);
                        r[2 * w] = v.x; r[2 * w + 1] = v.y;
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < HW; ++w) r[w] = ld_stream1(p + w);
                }
            }
            continue;
        }
        const uint32_t* p = reinterpret_cast<const uint32_t*>(kcodes + (t * C::RBK + grp * C::GB));
        if constexpr (C::GW % 4 == 0) {
#pragma unroll
            for (int w = 0; w < C::GW / 4; ++w) {
                const uint4 v = ld_stream4(p + 4 * w);
                rk[j * C::GW + 4 * w] = v.x; rk[j * C::GW + 4 * w + 1] = v.y;
                rk[j * C::GW + 4 * w + 2] = v.z; rk[j * C::GW + 4 * w + 3] = v.w;
            }
        } else if constexpr (C::GW % 2 == 0) {
#pragma unroll
            for (int w = 0; w < C::GW / 2; ++w) {
                const uint2 v = ld_stream2(p + 2 * w);
                rk[j * C::GW + 2 * w] = v.x; rk[j * C::GW + 2 * w + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int w = 0; w < C::GW; ++w) rk[j * C::GW + w] = ld_stream1(p + w);
        }
    }
}

// V row, norms (and QJL gamma) of token t0 + lane (clamped like fetch_k).
template <class C, bool QJL>
__device__ __forceinline__ void fetch_v(uint32_t (&rv)[C::VTW], uint32_t& rn, uint32_t& rg, uint32_t& rv2,
                                        const uint8_t* vcodes, const uint8_t* knb, const uint8_t* vnb,
                                        const uint8_t* gmb, uint32_t t0, uint32_t last, int lane, int nbk, int nbv) {
    uint32_t tl = t0 + lane;
    tl = tl < last ? tl : last;
    if constexpr (C::RBV % 16 == 0) {
        const uint4* vp = reinterpret_cast<const uint4*>(vcodes + tl * C::RBV);
#pragma unroll
        for (int w = 0; w < C::RBV / 16; ++w) {
            const uint4 v = ld_stream4(vp + w);
            rv[4 * w] = v.x; rv[4 * w + 1] = v.y; rv[4 * w + 2] = v.z; rv[4 * w + 3] = v.w;
        }
    } else {
        // 24-byte rows (3-bit values at d = 64): 8-byte loads keep every load aligned
        static_assert(C::RBV % 8 == 0, "V rows of whole 8-byte words");
        const uint2* vp = reinterpret_cast<const uint2*>(vcodes + tl * C::RBV);
#pragma unroll
        for (int w = 0; w < C::RBV / 8; ++w) {
            const uint2 v = ld_stream2(vp + w);
            rv[2 * w] = v.x; rv[2 * w + 1] = v.y;
        }
    }
    if constexpr (C::HALVES) {
        // rn: the K norms of the two halves, rg: the V norms (the one norm twice
        // for a cache with one norm block); no QJL with two norm blocks
        // (the norm arrays are only 2-byte aligned: two 16-bit loads per pair)
        const uint32_t k = nbk == 2 ? ld_stream_u16(knb + 4u * tl) | (ld_stream_u16(knb + 4u * tl + 2u) << 16)
                                    : ld_stream_u16(knb + 2u * tl) * 0x10001u;
        const uint32_t v = nbv == 2 ? ld_stream_u16(vnb + 4u * tl) | (ld_stream_u16(vnb + 4u * tl + 2u) << 16)
                                    : ld_stream_u16(vnb + 2u * tl) * 0x10001u;
        rn = k;
        rv2 = v;
        if constexpr (QJL) rg = ld_stream_u16(gmb + 2u * tl);
        return;
    }
    rn = ld_stream_u16(knb + 2u * tl) | (ld_stream_u16(vnb + 2u * tl) << 16);
    if constexpr (QJL) rg = ld_stream_u16(gmb + 2u * tl);
}

// QJL sign bytes of sub-tiles 0..3: token t0 + 16 j + n, the m/32 bytes of
// lane group grp (projections [m/4 grp, m/4 (grp + 1))), clamped like
// fetch_k.  Rows of m/8 bytes are only 4-byte aligned: dword loads at most.
__device__ __forceinline__ void fetch_q(uint32_t (&rq)[4][2], const uint8_t* qb, int m, uint32_t t0, uint32_t last,
                                        int n, int grp) {
    const uint32_t gbytes = (uint32_t)m >> 5, row = (uint32_t)m >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t t = t0 + 16 * j + n;
        t = t < last ? t : last;
        const uint8_t* p = qb + t * row + grp * gbytes;
        if (gbytes == 8 || gbytes == 4) {
            rq[j][0] = ld_stream1(p);
            rq[j][1] = gbytes == 8 ? ld_stream1(p + 4) : 0u;
        } else if (gbytes == 2) {
            rq[j][0] = ld_stream_u16(p);
            rq[j][1] = 0u;
        } else {
            // 1, 3, 5, 6 or 7 bytes (m = 32 or an odd multiple of 32): byte loads
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int b = 0; b < 7; ++b)
                if ((uint32_t)b < gbytes) w[b >> 2] |= (uint32_t)__builtin_nontemporal_load(p + b) << (8 * (b & 3));
            rq[j][0] = w[0];
            rq[j][1] = w[1];
        }
    }
}

// Query rows.  A sequence carries ncols query columns (its last ncols tokens,
// already in the cache) of hq heads; the rows of kv head kvh are its g heads
// in each column, vl = c * g + j for column c and head kvh * g + j, and a
// block takes G consecutive rows vl.  Row (b, c, h) is stored at index
// (b * ncols + c) * hq + h of the query, workspace and output arrays, and
// column c attends over the first ctx - (ncols - 1 - c) tokens (causal).
template <bool MQ>
__device__ __forceinline__ int64_t query_row(const AttnArgs& a, int b, int kvh, int vl) {
    if constexpr (!MQ) return (int64_t)b * a.hq + kvh * a.g + vl;  // one column
    const int c = vl / a.g;
    return ((int64_t)b * a.ncols + c) * a.hq + kvh * a.g + (vl - c * a.g);
}

// One instance per (D, KB, VB, QJL) and switch set: SPARSE = the sparse-V
// switch, MQ = more than one query column, GM = the row mode of the block:
//   GM = 8: eight query rows;
//   GM = 0: G < 8 rows (a runtime value).  In both, the 16 matrix-core
//           columns of a K step hold q_hi (columns 0..7) and q_lo (8..15) of
//           the same 8 rows, folded after the scores;
//   GM = 16: 9 to 16 rows (runtime G), one row per column: each K step runs
//           twice on the same looked-up operands, once against q_hi and once
//           against q_lo, into the same scores, so the lookups, softmax and V
//           sums of a tile serve twice the rows for 1.67x the matrix-core
//           work (2 x 32 K steps + 16 V steps against 32 + 16 per 8 rows).
// TWO: a cache with two norm blocks on either side (d = 256, the per-half
// layout of Cfg::HALVES; a side with one norm uses it for both halves).
template <int D, int KB, int VB, bool QJL, bool SPARSE, bool MQ, int GM, bool TWO>
__global__ __launch_bounds__(64 * split_waves(D, KB, VB, QJL))
__attribute__((amdgpu_waves_per_eu(split_waves(D, KB, VB, QJL) / 4)))
void split_kernel(AttnArgs a) {
    using C = Cfg<D, KB, VB, QJL, TWO>;
    constexpr bool R16 = GM == 16;
    static_assert(!R16 || split_rows16(D, QJL), "16-row blocks need d <= 128 and no QJL");
    const int G = GM == 8 ? 8 : a.heads_per_chunk;
    __shared__ __attribute__((aligned(16))) uint32_t smem[C::SMEM_DW];
    uint8_t* tab = reinterpret_cast<uint8_t*>(smem);
    uint32_t* waves_lds = smem + C::TABB / 4;
    uint4* qjlb = reinterpret_cast<uint4*>(waves_lds + C::NW * C::WAVE_DW);
    uint4* sigt = qjlb + 8 * 64;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.chunks, chunk = blockIdx.y - kvh * a.chunks;
    const int b = blockIdx.z;
    const int m = QJL ? a.kc.qjl_m : 0;
    // token indices fit 31 bits (ctx_cap * row bytes < 2^31 is checked on the host)
    const int cap = (int)a.ctx_cap;
    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int t_beg = split * (int)a.split_tokens;
    const int t_end = (t_beg + (int)a.split_tokens < ctx) ? t_beg + (int)a.split_tokens : ctx;
    const int vl0 = chunk * G;  // first row of this block (see query_row)
    // tokens a row may see: ctx for the last column, fewer for earlier ones
    const int ctx_min = MQ ? ctx - (a.ncols - 1 - vl0 / a.g) : ctx;  // the block's first row sees the fewest
    const int64_t kvrow = ((int64_t)b * a.hkv + kvh) * a.ctx_cap;
    const uint8_t* kcodes = a.k_codes + kvrow * C::RBK;
    const uint8_t* vcodes = a.v_codes + kvrow * C::RBV;
    // norm blocks per vector (two only with HALVES), their scale sqrt(blocks)
    const int nbk = C::HALVES ? a.kc.norm_blocks : 1, nbv = C::HALVES ? a.vc.norm_blocks : 1;
    const float bsk = nbk == 2 ? 1.41421356237309505f : 1.0f, bsv = nbv == 2 ? 1.41421356237309505f : 1.0f;
    const uint8_t* knb = reinterpret_cast<const uint8_t*>(a.k_norms + kvrow * nbk);
    const uint8_t* vnb = reinterpret_cast<const uint8_t*>(a.v_norms + kvrow * nbv);
    const uint8_t* gmb = QJL ? reinterpret_cast<const uint8_t*>(a.k_gamma + kvrow) : nullptr;
    const uint32_t last = t_end > 0 ? (uint32_t)(t_end - 1) : 0u;

    // This chunk's query rows are rotated here (the Q-side transform): lane
    // group hl = wave * QVPW + lane / QLPV of the first waves holds dims
    // [8 gl, 8 gl + 8) of row vl0 + hl.  Their loads go out first, so the
    // transform waits for them alone, then the first tile's loads.
    constexpr int QLPV = D / 8, QVPW = 64 / QLPV;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const bool qwave = wave_u * QVPW < G;
    const int qgl = lane & (QLPV - 1), qhl = wave_u * QVPW + lane / QLPV;
    float qx[8];
    if (qwave) {
        if (qhl < G) {
            const int64_t e0 = query_row<MQ>(a, b, kvh, vl0 + qhl) * D + qgl * 8;
            if (a.q_dtype == TQ_F32) load8<0>(static_cast<const float*>(a.q) + e0, qx);
            else if (a.q_dtype == TQ_F16) load8<1>(static_cast<const uint16_t*>(a.q) + e0, qx);
            else load8<2>(static_cast<const uint16_t*>(a.q) + e0, qx);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[e] = 0.0f;
        }
    }
    // first tile's loads go out before the tables are built
    int t0 = t_beg + wave_u * 64;
    constexpr bool KDB = C::KDB;
    constexpr int KBUF = KDB ? 2 : 1;  // K code buffers: with two, a tile's K codes are loaded one tile ahead
    uint32_t rk[KBUF][4 * C::GW];
    uint32_t rv[C::VTW], rn = 0, rg = 0, rv2 = 0;
    // QJL: the sign bytes of a tile, loaded a whole tile ahead (see kphase)
    uint32_t rq[4][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
    const uint8_t* qjb = QJL ? a.k_qjl + kvrow * (m >> 3) : nullptr;
    if (t0 < t_end) {
        fetch_k<C>(rk[0], kcodes, (uint32_t)t0, last, n, grp);
        fetch_v<C, QJL>(rv, rn, rg, rv2, vcodes, knb, vnb, gmb, (uint32_t)t0, last, lane, nbk, nbv);
        if constexpr (QJL) fetch_q(rq, qjb, m, (uint32_t)t0, last, n, grp);
    }

    // centroids once into LDS, then every table row is written as 16-byte
    // chunks that repeat one entry (one chunk covers 16 / entry-size slices)
    __shared__ float cent[32];  // [0, 16): 16 * c_K, [16, 32): c_V
    if (tid < (1 << KB)) cent[tid] = 16.0f * a.kc.centroid[tid];
    if (tid >= 16 && tid < 16 + (1 << VB)) cent[tid] = a.vc.centroid[tid - 16];
    // rotated queries qr[hl][dim] = (scale log2(e) / d) H(D_K q), in the wave
    // areas (free until the tile loop)
    float* qr = reinterpret_cast<float*>(waves_lds);
    if (qwave) {
        const uint32_t sbits = (a.kc.sign_mask[qgl >> 2] >> ((qgl & 3) * 8)) & 0xFFu;
#pragma unroll
        for (int e = 0; e < 8; ++e) qx[e] = as_f(as_u(qx[e]) ^ (((sbits >> e) & 1u) << 31));
        fwht<QLPV>(qx, qgl);
        if constexpr (D == 64) {
            if (a.kc.rotation == TQ_ROT_DOUBLE) second_pass<QLPV>(qx, qgl, a.kc.sign_mask3);
        }
        float qs = a.scale * kLog2e / (float)D;
        if (a.score_mode != 0 && qhl < G) {
            const int nr = MQ ? ctx - (a.ncols - 1 - (vl0 + qhl) / a.g) : ctx;  // tokens this row attends over
            qs *= score_factor(a, nr > 0 ? nr : 0);
        }
        if (qhl < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qr[qhl * D + qgl * 8 + e] = qx[e] * qs;
        }
    }
    __syncthreads();
    // one item per (row, table): its entry is computed once and written as the
    // row's NCI 16-byte chunks, chunk (c + tid) % NCI in step c, so the 16
    // lanes of a write pass (distinct rows) fall on distinct banks.  Split: K
    // rows then V rows, 16 chunks each; shared: row u's chunks 0..7 repeat the
    // K entry of u and chunks 8..15 the V entry.
    constexpr int NCI = C::SPLIT ? 16 : 8;  // chunks per item
    constexpr int NITEMS = C::SPLIT ? C::KROWS + C::VROWS : 2 * (C::TABB / 256);
    for (int i = tid; i < NITEMS; i += C::NT) {
        bool is_k;
        int u, dst;
        if constexpr (C::SPLIT) {
            is_k = i < C::KROWS;
            u = is_k ? i : i - C::KROWS;
            dst = (is_k ? 0 : C::VBASE) + 256 * u;
        } else {
            u = i >> 1;
            is_k = (i & 1) == 0;
            dst = 256 * u + (is_k ? 0 : 128);
        }
        uint32_t w[4] = {0u, 0u, 0u, 0u};  // one entry (K: hi halves then lo halves; V: halves)
        bool live;
        if (is_k) {
            live = u < C::KROWS;
#pragma unroll
            for (int p = 0; p < C::KE; p += 2) {
                const float c0 = cent[(u >> (KB * p)) & ((1 << KB) - 1)];
                const float c1 = cent[(u >> (KB * (p + 1))) & ((1 << KB) - 1)];
                const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
                w[p / 2] = pack_half2((float)h0, (float)h1);
                w[C::KE / 2 + p / 2] = pack_half2(c0 - (float)h0, c1 - (float)h1);
            }
        } else {
            live = u < C::VROWS;
#pragma unroll
            for (int p = 0; p < C::VT; p += 2)
                w[p / 2] = pack_half2(cent[16 + ((u >> (VB * p)) & ((1 << VB) - 1))],
                                      cent[16 + ((u >> (VB * (p + 1))) & ((1 << VB) - 1))]);
        }
        const int eb = is_k ? C::KENT : C::VENT;  // entry bytes
        uint4 v;
        if (eb == 4) v = make_uint4(w[0], w[0], w[0], w[0]);
        else if (eb == 8) v = make_uint4(w[0], w[1], w[0], w[1]);
        else v = make_uint4(w[0], w[1], w[2], w[3]);
        if (live) {
#pragma unroll
            for (int c = 0; c < NCI; ++c)
                *reinterpret_cast<uint4*>(tab + dst + 16 * ((c + tid) & (NCI - 1))) = v;
        }
    }
    if constexpr (QJL) {
        _Float16* st = reinterpret_cast<_Float16*>(sigt);
        for (int e = tid; e < 256 * 8; e += C::NT) st[e] = ((e >> 3) >> (e & 7)) & 1 ? (_Float16)1.0f : (_Float16)(-1.0f);
    }

    // K-side B operands: column n holds q_hi (n < 8) or q_lo (n >= 8) of head
    // n % 8 (zero beyond G), all heads scaled by one power of two, with the dims
    // of K step ks in the order of the A entries (KE = 2: d0 d1 d0 d1 d2 d3 d2 d3;
    // KE = 4: d0 d1 d2 d3 d0 d1 d2 d3); likewise the QJL projection.  With 16
    // rows, column n is head n: q_hi in bq, q_lo in bql.
    const int hh = R16 ? n : (n & 7);
    const bool lo_col = !R16 && n >= 8, head_ok = hh < G;
    const int ctx_row = MQ ? ctx - (a.ncols - 1 - (vl0 + hh) / a.g) : ctx;  // tokens row hh may see
    half8_t bq[C::KSTEPS];
    half8_t bql[R16 ? C::KSTEPS : 1];
    float qinv;
    {
        float qv[C::KSTEPS][4];
        float amax = 0.0f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = C::HALVES ? (ks < C::KSTEPS / 2 ? 0 : D / 2) + grp * (C::DG / 2) + 4 * (ks % (C::KSTEPS / 2)) + i
                                          : grp * C::DG + 4 * ks + i;
                const float x = qr[(head_ok ? hh : 0) * D + dim];
                qv[ks][i] = head_ok ? x : 0.0f;
                amax = fmaxf(amax, fabsf(qv[ks][i]));
            }
        const float* qp = a.qproj + query_row<MQ>(a, b, kvh, vl0 + (head_ok ? hh : 0)) * m;
        if constexpr (QJL) {
            for (int ks = 0; ks < (m >> 5); ++ks)
                for (int j = 0; j < 8; ++j)
                    amax = fmaxf(amax, head_ok ? fabsf(qp[grp * (m >> 2) + 8 * ks + j]) : 0.0f);
        }
        amax = wave_max(amax);
        float sc = 1.0f;
        if (amax > 0.0f && isfinite(amax)) {
            int e;
            frexpf(amax, &e);
            sc = ldexpf(1.0f, 15 - e);
        }
        qinv = 1.0f / (16.0f * sc);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            _Float16 x[4], xl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = qv[ks][i] * sc;
                const _Float16 hi = (_Float16)v;
                xl[i] = (_Float16)(v - (float)hi);
                x[i] = lo_col ? xl[i] : hi;
            }
#pragma unroll
            // the q_lo operands are zero on the c_lo slots: the c_lo * q_lo product
            // (below 2^-22 of the score) is left out, and zero operands cost the
            // matrix cores less energy
            for (int e = 0; e < 8; ++e) {
                const bool lo_slot = C::KE == 2 ? (e & 2) != 0 : (e & 4) != 0;
                const int di = C::KE == 2 ? (e >> 2) * 2 + (e & 1) : e & 3;
                bq[ks][e] = (lo_col && lo_slot) ? (_Float16)0.0f : x[di];
                if constexpr (R16) bql[ks][e] = lo_slot ? (_Float16)0.0f : xl[di];
            }
        }
        if constexpr (QJL) {
            if (wave == 0) {
                for (int ks = 0; ks < (m >> 5); ++ks) {
                    half8_t x8;
                    for (int j = 0; j < 8; ++j) {
                        // the sign products are scaled by 16*gamma later, so by sc only
                        const float v = (head_ok ? qp[grp * (m >> 2) + 8 * ks + j] : 0.0f) * sc;
                        const _Float16 hi = (_Float16)v;
                        x8[j] = lo_col ? (_Float16)(v - (float)hi) : hi;
                    }
                    qjlb[ks * 64 + lane] = __builtin_bit_cast(uint4, x8);
                }
            }
        }
    }
    uint32_t* vt = waves_lds + wave * C::WAVE_DW;                      // [VTW + 1][VSTR] dword-major V tile
    float* hfac = reinterpret_cast<float*>(vt + (C::VTW + 1) * C::VSTR);  // [16] per-head rescale factors
    float* knq = hfac + 16;                                             // [64] K norm * query scale
    float* vnl = knq + 64;                                              // [64] V norm * weight scale
    float* gml = vnl + 64;                                              // [64] QJL gamma
    float* knq1 = gml + 64;                                             // HALVES: [64] second-half K norm * query scale
    float* vnl1 = knq1 + 64;                                            // HALVES: [64] second-half V norm * weight scale
    __syncthreads();  // every wave has read qr before the wave areas are reused
    vt[C::VTW * C::VSTR + lane] = 0u;
    __syncthreads();
    // this lane's table slices (byte offsets inside a row)
    const uint32_t koff = (uint32_t)(lane % C::KSL) * C::KENT;
    const uint32_t voff = C::VOFF0 + (uint32_t)(lane % C::VSL) * C::VENT;

    constexpr bool sparse = SPARSE;
    float m_ref = -INFINITY, l_lane = 0.0f;  // head n's reference max / this lane's partial sum
    // V sums D[nb][i]: head 4*grp + i, dim NB*n + nb, in units of 2^wsh
    floatx4_t vacc[C::NB];
#pragma unroll
    for (int q = 0; q < C::NB; ++q) vacc[q] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // HALVES: the second half's K sums of the tile, its V norm (scaled like
    // vnf) and its V-side A operands
    floatx4_t sacc1[4];
    float vn1f = 0.0f;
    uint32_t wa1[2][4];
    int vref = -200;                 // reference V-norm exponent: norms < 2^vref
    float vlim = 0.0f, vsc = 0.0f;   // 2^vref, 2^wsh with wsh = 15 - kTauLog2 - vref
    const int pbit = C::PIECE * n;   // this lane's V field inside a row
    const int pw0 = pbit >> 5, psh = pbit & 31;

    // Software pipeline over this wave's tiles: iteration i stages tile i, runs
    // its K scores on the matrix cores in the same basic block as the V sums of
    // tile i-1 (so the matrix-core and VALU/LDS work of the two overlap), then
    // exponentiates tile i.  Every stage below is inlined at each use.
    auto wave_sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // stage tile t0 (lane <-> token) and prefetch the next tile's V row and
    // norms (and, with two K buffers, its K codes into buffer nxt)
    auto stage = [&](float& vnf, auto nxtc) __attribute__((always_inline)) -> bool {
        constexpr int nxt = decltype(nxtc)::value % KBUF;
        const int rem = t_end - t0;
        const bool lane_valid = lane < rem;
#pragma unroll
        for (int w = 0; w < C::VTW; ++w) vt[w * C::VSTR + lane] = rv[w];
        float vmx;  // the larger V norm of the token
        if constexpr (C::HALVES) {
            knq[lane] = half_bits_to_float(rn & 0xFFFFu) * (qinv * bsk);
            knq1[lane] = half_bits_to_float(rn >> 16) * (qinv * bsk);
            vnf = half_bits_to_float(rv2 & 0xFFFFu) * bsv;
            vn1f = half_bits_to_float(rv2 >> 16) * bsv;
            vnl1[lane] = vn1f * vsc;
            vmx = fmaxf(vnf, vn1f);
        } else {
            vnf = half_bits_to_float(rn >> 16);
            knq[lane] = half_bits_to_float(rn & 0xFFFFu) * qinv;
            vmx = vnf;
        }
        if constexpr (QJL) gml[lane] = 16.0f * half_bits_to_float(rg);
        vnl[lane] = vnf * vsc;
        // prefetch (clamped to the split: past its end this re-reads the last token)
        fetch_v<C, QJL>(rv, rn, rg, rv2, vcodes, knb, vnb, gmb, (uint32_t)(t0 + 64 * C::NW), last, lane, nbk, nbv);
        if constexpr (KDB) fetch_k<C>(rk[nxt], kcodes, (uint32_t)(t0 + 64 * C::NW), last, n, grp);
        // a V norm at or above the reference is handled by the rare rescale
        return __builtin_amdgcn_ballot_w64(lane_valid && vmx >= vlim) != 0;
    };
    // K scores of tile t0 (16 tokens x 16 columns per sub-tile), then prefetch the next tile's K codes
    // (K codes from buffer cur; with one buffer the next tile's codes are loaded after the lookups)
    auto kphase = [&](floatx4_t (&sacc)[4], auto curc) __attribute__((always_inline)) {
        constexpr int cur = decltype(curc)::value % KBUF;
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (C::HALVES) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sacc1[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // step s = (sub-tile j, K step ks); the table lookups of step
        // s + kKLookahead are issued before the matrix-core op of step s, and
        // scheduling barriers keep that order
        constexpr int NS = 4 * C::KSTEPS;
        uint32_t aw[NS][4];
        auto look = [&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value, j = s / C::KSTEPS, ks = s % C::KSTEPS;
#pragma unroll
            for (int u = 0; u < C::LPS; ++u) {
                const int bit = (4 * ks + u * C::KE) * KB;
                uint32_t addr;
                if constexpr (C::KLU == 8) {
                    // row offset = index * 256 + koff: one byte permute
                    const uint32_t w = rk[cur][j * C::GW + (bit >> 5)];
                    addr = __builtin_amdgcn_perm(w, koff, 0x0C020000u | ((uint32_t)(4 + ((bit >> 3) & 3)) << 8));
                } else {
                    addr = field_at<C::KLU>(rk[cur] + j * C::GW, bit) * 256u + koff;
                }
                lds_read<C::KENT / 4>(aw[s] + u * (C::KENT / 4), tab + addr);
            }
        };
        static_for<kKLookahead>(look);
        static_for<NS>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value, j = s / C::KSTEPS, ks = s % C::KSTEPS;
            if constexpr (s + kKLookahead < NS) look(std::integral_constant<int, s + kKLookahead>{});
            __builtin_amdgcn_sched_barrier(0);
            const half8_t ak = as_half8(make_uint4(aw[s][0], aw[s][1], aw[s][2], aw[s][3]));
            // the K steps of the second half accumulate apart (HALVES)
            floatx4_t& acc = (C::HALVES && ks >= C::KSTEPS / 2) ? sacc1[j] : sacc[j];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bq[ks], acc, 0, 0, 0);
            if constexpr (R16) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bql[ks], acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (!KDB) fetch_k<C>(rk[cur], kcodes, (uint32_t)(t0 + 64 * C::NW), last, n, grp);
        if constexpr (QJL) {
            // A = the +-1 signs of token 16j + n, accumulated apart and scaled
            // by the token's 16*gamma in float32 before joining the scores.
            // The sign bytes came with the previous tile; the next tile's go
            // out once these are used.  Step ks outer (one uniform branch and
            // one read of the projected query per step), the four sub-tiles'
            // independent chains inner.
            const int nks = m >> 5;
            floatx4_t qacc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) qacc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks < nks) {
                    const half8_t bqj = as_half8(qjlb[ks * 64 + lane]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t byte = (rq[j][ks >> 2] >> (8 * (ks & 3))) & 0xFFu;
                        qacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(sigt[byte]), bqj, qacc[j], 0, 0, 0);
                    }
                }
            }
            // row v of sub-tile j's result is token 16j + 4grp + v
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 g4 = *reinterpret_cast<const float4*>(gml + 16 * j + 4 * grp);
                sacc[j][0] = fmaf(qacc[j][0], g4.x, sacc[j][0]);
                sacc[j][1] = fmaf(qacc[j][1], g4.y, sacc[j][1]);
                sacc[j][2] = fmaf(qacc[j][2], g4.z, sacc[j][2]);
                sacc[j][3] = fmaf(qacc[j][3], g4.w, sacc[j][3]);
            }
            fetch_q(rq, qjb, m, (uint32_t)(t0 + 64 * C::NW), last, n, grp);
        }
        // column h + 8 holds the q_lo part of head h: add the two halves of each row
        if constexpr (!R16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) sacc[j][v] += xor_lane<8>(sacc[j][v]);
            if constexpr (C::HALVES) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) sacc1[j][v] += xor_lane<8>(sacc1[j][v]);
            }
        }
    };
    // scores of tile t0 relative to the reference max, the rare rescale, and the
    // V-side A operands: half weights p * |v| * 2^wsh (K order: sub-tile pairs
    // (2 s2, 2 s2 + 1), tokens 4grp + v), row = head n
    auto softmax = [&](const floatx4_t (&sacc)[4], bool vraise, float vnf, uint32_t (&wa)[2][4])
        __attribute__((always_inline)) {
        const int rem = t_end - t0;
        float dsc[4][4];
        float lmax = -INFINITY;
        // this lane's row sees tokens below row_end; every row of the block
        // sees the whole tile unless it reaches past ctx_min or t_end
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 kq = *reinterpret_cast<const float4*>(knq + 16 * j + 4 * grp);
            dsc[j][0] = fmaf(sacc[j][0], kq.x, -m_ref);
            dsc[j][1] = fmaf(sacc[j][1], kq.y, -m_ref);
            dsc[j][2] = fmaf(sacc[j][2], kq.z, -m_ref);
            dsc[j][3] = fmaf(sacc[j][3], kq.w, -m_ref);
            if constexpr (C::HALVES) {
                const float4 kq1 = *reinterpret_cast<const float4*>(knq1 + 16 * j + 4 * grp);
                dsc[j][0] = fmaf(sacc1[j][0], kq1.x, dsc[j][0]);
                dsc[j][1] = fmaf(sacc1[j][1], kq1.y, dsc[j][1]);
                dsc[j][2] = fmaf(sacc1[j][2], kq1.z, dsc[j][2]);
                dsc[j][3] = fmaf(sacc1[j][3], kq1.w, dsc[j][3]);
            }
        }
        // token 16j + 4grp + v is valid iff 16j + v < lim
        int lim;
        bool partial;
        if constexpr (MQ) {
            const int row_end = ctx_row < t_end ? ctx_row : t_end;
            lim = row_end - t0 - 4 * grp;
            partial = (ctx_min < t_end ? ctx_min : t_end) - t0 < 64;
        } else {
            lim = rem - 4 * grp;
            partial = rem < 64;
        }
        if (partial) {
            // keeps the compares inside this (last-tile) branch
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (16 * j + v >= lim) dsc[j][v] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) lmax = fmaxf(lmax, dsc[j][v]);
        if (__builtin_amdgcn_ballot_w64(lmax > kTauLog2) || vraise) {
            // rare: raise the V-norm reference and/or the reference max of every
            // head (to its tile max), rescaling the running sums
            float vfac = 1.0f;
            if (vraise) {
                const float vm = wave_max(lane < rem ? (C::HALVES ? fmaxf(vnf, vn1f) : vnf) : 0.0f);
                int e;
                frexpf(vm, &e);
                const int vnew = e + kVHeadroom;
                vfac = ldexpf(1.0f, vref - vnew);
                vref = vnew;
                vlim = ldexpf(1.0f, vref);
                vsc = ldexpf(1.0f, 15 - (int)kTauLog2 - vref);
                vnl[lane] = vnf * vsc;
                if constexpr (C::HALVES) vnl1[lane] = vn1f * vsc;
            }
            float sv[4][4], tmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 kq = *reinterpret_cast<const float4*>(knq + 16 * j + 4 * grp);
                const float kv[4] = {kq.x, kq.y, kq.z, kq.w};
                float kv1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (C::HALVES) {
                    const float4 kq1 = *reinterpret_cast<const float4*>(knq1 + 16 * j + 4 * grp);
                    kv1[0] = kq1.x; kv1[1] = kq1.y; kv1[2] = kq1.z; kv1[3] = kq1.w;
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float sk = C::HALVES ? fmaf(sacc1[j][v], kv1[v], sacc[j][v] * kv[v]) : sacc[j][v] * kv[v];
                    sv[j][v] = (16 * j + v < lim) ? sk : -INFINITY;
                    tmax = fmaxf(tmax, sv[j][v]);
                }
            }
            tmax = fmaxf(tmax, xor_lane<16>(tmax));
            tmax = fmaxf(tmax, xor_lane<32>(tmax));
            // a row that has seen no token yet (an early column of a
            // multi-query block) keeps max -inf and weight zero
            const float mnew = fmaxf(m_ref, tmax);
            const bool none = mnew == -INFINITY;
            const float alpha = none ? 1.0f : fast_exp2(m_ref - mnew);
            m_ref = mnew;
            l_lane *= alpha;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) dsc[j][v] = none ? -INFINITY : sv[j][v] - mnew;
            if (grp == 0) hfac[n] = alpha * vfac;
            wave_sync();
            const float4 f4 = *reinterpret_cast<const float4*>(hfac + 4 * grp);
#pragma unroll
            for (int q = 0; q < C::NB; ++q) {
                vacc[q][0] *= f4.x;
                vacc[q][1] *= f4.y;
                vacc[q][2] *= f4.z;
                vacc[q][3] *= f4.w;
            }
        }
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 vq = *reinterpret_cast<const float4*>(vnl + 16 * j + 4 * grp);
            const float p0 = fast_exp2(dsc[j][0]), p1 = fast_exp2(dsc[j][1]);
            const float p2 = fast_exp2(dsc[j][2]), p3 = fast_exp2(dsc[j][3]);
            psum += (p0 + p1) + (p2 + p3);
            wa[j >> 1][2 * (j & 1)] = pack_half2(p0 * vq.x, p1 * vq.y);
            wa[j >> 1][2 * (j & 1) + 1] = pack_half2(p2 * vq.z, p3 * vq.w);
            if constexpr (C::HALVES) {
                const float4 vq1 = *reinterpret_cast<const float4*>(vnl1 + 16 * j + 4 * grp);
                wa1[j >> 1][2 * (j & 1)] = pack_half2(p0 * vq1.x, p1 * vq1.y);
                wa1[j >> 1][2 * (j & 1) + 1] = pack_half2(p2 * vq1.z, p3 * vq1.w);
            }
        }
        l_lane += psum;
        if (sparse) {
            // sparse V: weights below 2^sparse_log2 of the reference max keep
            // their place in the sum above but add nothing to the V sums (the
            // reference max never exceeds the true one, so only weights below
            // the threshold of the true max are dropped)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t k0 = (dsc[j][0] < a.sparse_log2 ? 0u : 0xFFFFu) | (dsc[j][1] < a.sparse_log2 ? 0u : 0xFFFF0000u);
                const uint32_t k1 = (dsc[j][2] < a.sparse_log2 ? 0u : 0xFFFFu) | (dsc[j][3] < a.sparse_log2 ? 0u : 0xFFFF0000u);
                wa[j >> 1][2 * (j & 1)] &= k0;
                wa[j >> 1][2 * (j & 1) + 1] &= k1;
                if constexpr (C::HALVES) {
                    wa1[j >> 1][2 * (j & 1)] &= k0;
                    wa1[j >> 1][2 * (j & 1) + 1] &= k1;
                }
            }
        }
        // rows of heads >= G (with G <= 8 also the repeated rows 8..15) carry
        // zero weights (they are never read; zero operands cost the matrix
        // cores less energy)
        if (n >= G) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    wa[s2][w] = 0u;
                    if constexpr (C::HALVES) wa1[s2][w] = 0u;
                }
        }
    };
    // this lane's PIECE-bit field of the staged tile's tokens e = 4 jj + v (token
    // 32 s2 + 16 jj + 4 grp + v): fields of PK consecutive tokens share one word
    // when PIECE <= 16; otherwise pc holds the low 32 bits and ph the rest
    constexpr int PK = C::PIECE == 16 ? 2 : (C::PIECE == 8 ? 4 : 1);
    const uint32_t psel = C::PIECE == 16 ? (psh ? 0x07060302u : 0x05040100u)
                                         : (0x0C0C0400u | (uint32_t)(psh >> 3) | ((uint32_t)(4 + (psh >> 3)) << 8));
    auto vread = [&](uint32_t (&pc)[2][8], uint32_t (&ph)[2][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int tok = 32 * s2 + 16 * jj + 4 * grp;
                if constexpr (C::HALVES) {
                    // the lane's dims are [NB/2 n, NB/2 n + NB/2) of each half: two
                    // HB-bit fields, the first half's in the low bits of the piece
                    constexpr int HB = C::PIECE / 2;
                    constexpr uint32_t HM = HB == 32 ? 0xFFFFFFFFu : (1u << HB) - 1u;
                    const int b0 = HB * n, b1 = (D / 2) * VB + HB * n;
                    const uint4 x0 = *reinterpret_cast<const uint4*>(vt + (b0 >> 5) * C::VSTR + tok);
                    const uint4 x1 = *reinterpret_cast<const uint4*>(vt + (b1 >> 5) * C::VSTR + tok);
                    const uint32_t l0[4] = {x0.x, x0.y, x0.z, x0.w}, l1[4] = {x1.x, x1.y, x1.z, x1.w};
                    uint32_t h0[4], h1[4];
                    if constexpr (32 % HB != 0) {
                        // a field may cross into the next dword (the tile's last row is zero)
                        const uint4 y0 = *reinterpret_cast<const uint4*>(vt + ((b0 >> 5) + 1) * C::VSTR + tok);
                        const uint4 y1 = *reinterpret_cast<const uint4*>(vt + ((b1 >> 5) + 1) * C::VSTR + tok);
                        const uint32_t u0[4] = {y0.x, y0.y, y0.z, y0.w}, u1[4] = {y1.x, y1.y, y1.z, y1.w};
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            h0[v] = __builtin_amdgcn_alignbit(u0[v], l0[v], b0 & 31) & HM;
                            h1[v] = __builtin_amdgcn_alignbit(u1[v], l1[v], b1 & 31) & HM;
                        }
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            h0[v] = (l0[v] >> (b0 & 31)) & HM;
                            h1[v] = (l1[v] >> (b1 & 31)) & HM;
                        }
                    }
                    if constexpr (PK == 2) {
                        pc[s2][2 * jj] = (h0[0] | (h1[0] << HB)) | ((h0[1] | (h1[1] << HB)) << 16);
                        pc[s2][2 * jj + 1] = (h0[2] | (h1[2] << HB)) | ((h0[3] | (h1[3] << HB)) << 16);
                    } else if constexpr (C::PIECE == 32) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) pc[s2][4 * jj + v] = h0[v] | (h1[v] << HB);
                    } else {
                        static_assert(C::PIECE > 32 && C::PIECE <= 64, "V piece of 33..64 bits");
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            pc[s2][4 * jj + v] = HB == 32 ? h0[v] : (h0[v] | (h1[v] << HB));
                            ph[s2][4 * jj + v] = HB == 32 ? h1[v] : (h1[v] >> (32 - HB));
                        }
                    }
                    continue;
                }
                const uint4 x = *reinterpret_cast<const uint4*>(vt + pw0 * C::VSTR + tok);
                const uint32_t lo[4] = {x.x, x.y, x.z, x.w};
                if constexpr (PK == 2) {
                    // the lane's halves of tokens (v, v + 1) side by side
                    pc[s2][2 * jj] = __builtin_amdgcn_perm(lo[1], lo[0], psel);
                    pc[s2][2 * jj + 1] = __builtin_amdgcn_perm(lo[3], lo[2], psel);
                } else if constexpr (PK == 4) {
                    // the lane's bytes of tokens v = 0..3
                    pc[s2][jj] = __builtin_amdgcn_perm(lo[1], lo[0], psel) |
                                 (__builtin_amdgcn_perm(lo[3], lo[2], psel) << 16);
                } else if constexpr (C::PIECE <= 32 && 32 % C::PIECE == 0) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) pc[s2][4 * jj + v] = lo[v] >> psh;
                } else {
                    const uint4 y = *reinterpret_cast<const uint4*>(vt + (pw0 + 1) * C::VSTR + tok);
                    const uint32_t hi[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        pc[s2][4 * jj + v] = __builtin_amdgcn_alignbit(hi[v], lo[v], psh);
                        ph[s2][4 * jj + v] = hi[v] >> psh;  // psh < 32; only read when PIECE > 32
                    }
                }
            }
    };
    // V sums of one tile on matrix cores from its pieces and weights
    auto vphase = [&](const uint32_t (&pc)[2][8], const uint32_t (&ph)[2][8], const uint32_t (&wa)[2][4])
        __attribute__((always_inline)) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            // sparse V: a 32-token step whose weights are all dropped is skipped
            // (its table lookups and matrix-core ops)
            if (sparse && !__builtin_amdgcn_ballot_w64((wa[s2][0] | wa[s2][1] | wa[s2][2] | wa[s2][3] |
                                                        (C::HALVES ? wa1[s2][0] | wa1[s2][1] | wa1[s2][2] | wa1[s2][3]
                                                                   : 0u)) != 0u))
                continue;
            const half8_t aw0 = as_half8(make_uint4(wa[s2][0], wa[s2][1], wa[s2][2], wa[s2][3]));
            const half8_t aw1 = C::HALVES ? as_half8(make_uint4(wa1[s2][0], wa1[s2][1], wa1[s2][2], wa1[s2][3])) : aw0;
#pragma unroll
            for (int k = 0; k < C::VLK; ++k) {
                const int bit = k * C::VLB;
                uint32_t ent[8][C::VENTW];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t addr;
                    if constexpr (C::VLB == 8) {
                        // byte-aligned index: row offset = index * 256 + voff by one byte permute
                        const int pos = (PK > 1 ? (e % PK) * C::PIECE : 0) + bit;  // bit position in its word
                        const uint32_t w = PK > 1 ? pc[s2][e / PK] : (pos < 32 ? pc[s2][e] : ph[s2][e]);
                        addr = __builtin_amdgcn_perm(w, voff, 0x0C020000u | ((uint32_t)(4 + ((pos >> 3) & 3)) << 8));
                    } else {
                        uint32_t idx;
                        if constexpr (PK > 1) {
                            idx = (pc[s2][e / PK] >> ((e % PK) * C::PIECE + bit)) & ((1u << C::VLB) - 1u);
                        } else if constexpr (C::PIECE <= 32) {
                            idx = (pc[s2][e] >> bit) & ((1u << C::VLB) - 1u);
                        } else {
                            const uint64_t x = ((uint64_t)ph[s2][e] << 32) | pc[s2][e];
                            idx = (uint32_t)(x >> bit) & ((1u << C::VLB) - 1u);
                        }
                        addr = idx * 256u + voff;
                    }
                    lds_read<C::VENTW>(ent[e], tab + C::VIMM + addr);
                }
#pragma unroll
                for (int h = 0; h < C::VT; ++h) {
                    const uint32_t sel = (h & 1) ? 0x07060302u : 0x05040100u;
                    const uint4 bq = make_uint4(__builtin_amdgcn_perm(ent[1][h >> 1], ent[0][h >> 1], sel),
                                                __builtin_amdgcn_perm(ent[3][h >> 1], ent[2][h >> 1], sel),
                                                __builtin_amdgcn_perm(ent[5][h >> 1], ent[4][h >> 1], sel),
                                                __builtin_amdgcn_perm(ent[7][h >> 1], ent[6][h >> 1], sel));
                    const int nb = k * C::VT + h;
                    // with HALVES, columns nb >= NB/2 are second-half dims (their own V norms)
                    const half8_t aw = (C::HALVES && nb >= C::NB / 2) ? aw1 : aw0;
                    vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_half8(bq), vacc[nb], 0, 0, 0);
                }
            }
        }
    };

    if (t0 < t_end) {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        uint32_t wa[2][4], pc[2][8], ph[2][8];
        floatx4_t sacc[4];
        float vnf;
        bool vraise = stage(vnf, I1{});
        wave_sync();
        kphase(sacc, I0{});
        softmax(sacc, vraise, vnf, wa);
        t0 += 64 * C::NW;
        // one tile: its K codes are in buffer cur, the next tile's go to the other
        auto tile = [&](auto curc) __attribute__((always_inline)) {
            vread(pc, ph);  // previous tile, before this tile overwrites the staging area
            wave_sync();
            vraise = stage(vnf, std::integral_constant<int, 1 - decltype(curc)::value>{});
            wave_sync();
            kphase(sacc, curc);
            vphase(pc, ph, wa);  // previous tile's V sums, before this tile's rescale
            softmax(sacc, vraise, vnf, wa);
            t0 += 64 * C::NW;
        };
        if constexpr (KDB) {
            while (t0 < t_end) {
                tile(I1{});
                if (t0 >= t_end) break;
                tile(I0{});
            }
        } else {
            while (t0 < t_end) tile(I0{});
        }
        vread(pc, ph);
        vphase(pc, ph, wa);
    }

    // block merge of the waves (V sums back to true units)
    const float wunit = ldexpf(1.0f, vref - 15 + (int)kTauLog2);
    float l_head = l_lane + xor_lane<16>(l_lane);
    l_head += xor_lane<32>(l_head);
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(smem);  // [NW][G][D + 2]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float mh = bcast_lane(m_ref, h);
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
            float* rr = mrg + (wave * G + h) * (D + 2) + 2;
#pragma unroll
            for (int q = 0; q < C::NB; ++q) {
                // the dim of column n of V sum q (see the V pieces)
                const int dim = C::HALVES ? (q < C::NB / 2 ? 0 : D / 2) + (C::NB / 2) * n + (q % (C::NB / 2))
                                          : C::NB * n + q;
                rr[dim] = vacc[q][i] * wunit;
            }
        }
    }
    __syncthreads();
    // per head: the block max and each wave's factor 2^(m_w - max) (0 for a
    // head no wave has seen), once, then every value of the head
    float* fac = mrg + C::NW * G * (D + 2);  // [G][NW + 1]: factors, then the max
    if (tid < G) {
        const int h = tid;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) mx = fmaxf(mx, mrg[(w * G + h) * (D + 2)]);
#pragma unroll
        for (int w = 0; w < C::NW; ++w)
            fac[h * (C::NW + 1) + w] = mx == -INFINITY ? 0.0f : exp2f(mrg[(w * G + h) * (D + 2)] - mx);
        fac[h * (C::NW + 1) + C::NW] = mx;
    }
    __syncthreads();
    for (int e = tid; e < G * (D + 2); e += C::NT) {
        const int h = e / (D + 2), i = e - h * (D + 2);
        const float* fh = fac + h * (C::NW + 1);
        float val;
        if (i == 0) {
            val = fh[C::NW];
        } else {
            val = 0.0f;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) val = fmaf(mrg[(w * G + h) * (D + 2) + i], fh[w], val);
        }
        a.part[(query_row<MQ>(a, b, kvh, vl0 + h) * a.splits + split) * (D + 2) + i] = val;
    }
}

// --------------------------------------------------------------- combine ----
// One lane group of D/8 lanes per (batch, query head), lane gl holding dims
// [8 gl, 8 gl + 8) as in the encoder's transform layout: the log-sum-exp merge
// of the head's split partials runs in registers, then the inverse transform
// D_V H(.) / d through lane exchanges.  No LDS and no barriers.
//
// combine_head merges the splits of head bh into the running state (mx, L, x)
// (rotated domain, log2 units) and writes the output row when `store`.
template <int D>
__device__ __forceinline__ void combine_head(const AttnArgs& a, int64_t bh, int gl, bool store, float mx, float L,
                                             float (&x)[8]) {
    constexpr int LPV = D / 8;
    const int S = a.splits;
    const float* p = a.part + bh * S * (D + 2);
    // online merge over chunks of four splits: the loads of a chunk go out
    // together, its max raises the running one and rescales the sums
    for (int s0 = 0; s0 < S; s0 += 4) {
        float mc[4], lc[4], vc[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool live = s0 + u < S;
            const float* ps = p + (int64_t)(live ? s0 + u : S - 1) * (D + 2);
            mc[u] = ps[0];
            lc[u] = ps[1];
            // dims 8 gl .. 8 gl + 7 of the split's sums (8-byte aligned: D + 2 is even)
            const float2* v2 = reinterpret_cast<const float2*>(ps + 2 + 8 * gl);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float2 v = v2[k];
                vc[u][2 * k] = v.x;
                vc[u][2 * k + 1] = v.y;
            }
            if (!live) mc[u] = -INFINITY;  // a repeated split weighs zero
        }
        const float nm = fmaxf(fmaxf(mx, fmaxf(mc[0], mc[1])), fmaxf(mc[2], mc[3]));
        if (nm != -INFINITY) {
            // a split with max -inf (no tokens) has zero sums and weighs exp2(-inf) = 0
            const float f0 = exp2f(mx - nm);
            L *= f0;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= f0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = exp2f(mc[u] - nm);
                L = fmaf(lc[u], f, L);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = fmaf(vc[u][e], f, x[e]);
            }
            mx = nm;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = L > 0.0f ? x[e] / L : 0.0f;
    // inverse rotation: D_V R(x) / d (R = H, or H D3 H / sqrt(d))
    fwht<LPV>(x, gl);
    if constexpr (D == 64) {
        if (a.vc.rotation == TQ_ROT_DOUBLE) second_pass<LPV>(x, gl, a.vc.sign_mask3);
    }
    const uint32_t sbits = (a.vc.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = as_f(as_u(x[e] * (1.0f / (float)D)) ^ (((sbits >> e) & 1u) << 31));
    if (store) {
        float4* o = reinterpret_cast<float4*>(a.out + bh * D + 8 * gl);
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
    constexpr int LPV = D / 8, HPB = 256 / LPV;  // lanes per head, heads per block
    const int tid = threadIdx.x, gl = tid & (LPV - 1);
    const int heads = a.batch * a.ncols * a.hq;
    const int bh = blockIdx.x * HPB + tid / LPV;
    const bool valid = bh < heads;  // uniform inside a lane group
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    combine_head<D>(a, valid ? bh : 0, gl, valid, -INFINITY, 0.0f, x);
}

// ---------------------------------------------------------------- window ----
// Residual window: the most recent tokens of a sequence kept exact, which join
// the softmax after the packed ones (the V3 cache of the PyTorch reproduction,
// "[GitHub 탐방] TurboQuant 3-bit KV 캐시 압축", "실험 설계" and "결과 — 피크
// VRAM").  One block of 4 waves per (batch, query head), XCD-aware; a lane group of D/8
// lanes takes one token at a time, lane gl holding dims [8 gl, 8 gl + 8), and
// loads U tokens' rows before using any of them.  Each group runs an online
// softmax in the scan's log2 units; groups merge by lane exchanges, waves
// through LDS.  The window's weighted value sum y enters the merge with the
// head's split partials as x = H(D_V y), so that the final D_V H(.) / d returns
// y; this kernel then writes the output (it replaces the combine launch).
template <int D, int WDT>
__global__ __launch_bounds__(256) void window_kernel(AttnArgs a) {
    constexpr int LPV = D / 8, TPW = 64 / LPV;  // lanes per token, tokens per wave
    constexpr int U = 8;                        // tokens per lane group per round, loaded together
    constexpr int STEP = 4 * TPW;               // tokens per block pass (4 waves)
    __shared__ float mrg[4][D + 2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (LPV - 1), tg = lane / LPV;
    // One block per (batch, query head).  Workgroups are dealt round-robin to
    // the 8 XCDs, each with its own L2: block i serves (batch, kv head) unit
    // i mod U8 (U8 = units rounded up to a multiple of 8) and query head
    // i / U8 of its group, so the g heads that read one window share an XCD
    // and its L2.
    const int units = a.batch * a.hkv, u8 = (units + 7) & ~7;
    const int unit = blockIdx.x % u8, hl = blockIdx.x / u8;
    if (unit >= units) return;  // whole block: before any barrier
    const int b = unit / a.hkv, kvh = unit - b * a.hkv;
    const int h = kvh * a.g + hl;
    const int bh = b * a.hq + h;
    const int wl_raw = a.win_len[b];
    // the query's raw words now, converted after the first window loads are out
    uint4 qw0 = make_uint4(0u, 0u, 0u, 0u), qw1 = qw0;
    if (a.q_dtype == TQ_F32) {
        const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + (int64_t)bh * D + 8 * gl);
        qw0 = qp[0];
        qw1 = qp[1];
    } else {
        qw0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + (int64_t)bh * D + 8 * gl);
    }
    float q[8];
    bool qready = false;
    const float qs = a.scale * kLog2e;
    const int64_t wrow = ((int64_t)b * a.hkv + kvh) * a.win_cap;
    const char* kw = static_cast<const char*>(a.k_win);
    const char* vw = static_cast<const char*>(a.v_win);
    float m = -INFINITY, l = 0.0f, y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.0f;
    // Token of (round r, slot u) for this lane group: t0 + u * STEP with
    // t0 = r * U * STEP + wave * TPW + tg.  Row indices are clamped to the
    // capacity, so the first round's loads go out together with the window
    // length's and the query's; tokens at or past the length are masked.  The
    // lanes of one group share t0 and so their trip count: the in-group
    // reduction only reads active lanes.
    int wl = -1;
    for (int t0 = wave * TPW + tg;; t0 += U * STEP) {
        float k[U][8], v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int t = t0 + u * STEP;
            t = t < a.win_cap ? t : a.win_cap - 1;
            // the window dtype is a template argument: no branch between the
            // loads, so all 2U of them are in flight before the first use
            const int64_t off = ((wrow + t) * D + 8 * gl) * elem_bytes<WDT>();
            load8<WDT>(kw + off, k[u]);
            load8<WDT>(vw + off, v[u]);
        }
        if (wl < 0) wl = wl_raw < 0 ? 0 : (wl_raw > a.win_cap ? a.win_cap : wl_raw);
        if (!qready) {
            const uint32_t w[8] = {qw0.x, qw0.y, qw0.z, qw0.w, qw1.x, qw1.y, qw1.z, qw1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t hw = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                q[e] = a.q_dtype == TQ_F32 ? as_f(w[e]) : (a.q_dtype == TQ_F16 ? half_bits_to_float(hw) : as_f(hw << 16));
            }
            qready = true;
        }
        float sc[U], cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(q[e], k[u][e], dot);
            const float su = group_sum<LPV>(dot) * qs;  // every lane, then masked: no branch
            sc[u] = t0 + u * STEP < wl ? su : -INFINITY;
            cm = fmaxf(cm, sc[u]);
        }
        const float mn = fmaxf(m, cm);
        if (mn != -INFINITY) {
            const float f = exp2f(m - mn);
            l *= f;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = exp2f(sc[u] - mn);
                l += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = fmaf(p, v[u][e], y[e]);
            }
            m = mn;
        }
        if (t0 + U * STEP >= wl) break;
    }
    // merge (m, l, y) of two states; an empty state has m = -inf and zeros
    auto join = [&](float mo, float lo, const float (&yo)[8]) __attribute__((always_inline)) {
        const float mn = fmaxf(m, mo);
        if (mn != -INFINITY) {
            const float f = exp2f(m - mn), fo = exp2f(mo - mn);
            l = l * f + lo * fo;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] * f + yo[e] * fo;
            m = mn;
        }
    };
    // the TPW lane groups of the wave (lane bits above the group)
    auto merge_lanes = [&](auto mc) __attribute__((always_inline)) {
        constexpr int M = decltype(mc)::value;
        const float mo = xor_lane<M>(m), lo = xor_lane<M>(l);
        float yo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) yo[e] = xor_lane<M>(y[e]);
        join(mo, lo, yo);
    };
    if constexpr (TPW >= 8) merge_lanes(std::integral_constant<int, 8>{});
    if constexpr (TPW >= 4) merge_lanes(std::integral_constant<int, 16>{});
    merge_lanes(std::integral_constant<int, 32>{});
    // the 4 waves, through LDS
    if (tg == 0) {
        if (gl == 0) {
            mrg[wave][0] = m;
            mrg[wave][1] = l;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) mrg[wave][2 + 8 * gl + e] = y[e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        float yo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) yo[e] = mrg[w][2 + 8 * gl + e];
        join(mrg[w][0], mrg[w][1], yo);
    }
    // the window's share in the rotated domain, x = R(D_V y), then the merge
    // with the head's split partials and the output (every lane group of wave
    // 0 holds the merged state, up to the rounding order of its merges; group
    // 0's is the one stored)
    const uint32_t sbits = (a.vc.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = as_f(as_u(y[e]) ^ (((sbits >> e) & 1u) << 31));
    fwht<LPV>(y, gl);
    if constexpr (D == 64) {
        if (a.vc.rotation == TQ_ROT_DOUBLE) second_pass<LPV>(y, gl, a.vc.sign_mask3);
    }
    combine_head<D>(a, bh, gl, tg == 0, m, l, y);
}

template <int D, int KB, int VB, bool QJL, int GM, bool TWO>
void launch_split_g(const AttnArgs& a, hipStream_t s) {
    const dim3 grid(a.splits, a.hkv * a.chunks, a.batch);
    const dim3 block(64 * split_waves(D, KB, VB, QJL));
    const bool sparse = a.sparse_log2 > -INFINITY, mq = a.ncols > 1;
    if (sparse && mq)
        hipLaunchKernelGGL((split_kernel<D, KB, VB, QJL, true, true, GM, TWO>), grid, block, 0, s, a);
    else if (sparse)
        hipLaunchKernelGGL((split_kernel<D, KB, VB, QJL, true, false, GM, TWO>), grid, block, 0, s, a);
    else if (mq)
        hipLaunchKernelGGL((split_kernel<D, KB, VB, QJL, false, true, GM, TWO>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((split_kernel<D, KB, VB, QJL, false, false, GM, TWO>), grid, block, 0, s, a);
}

template <int D, int KB, int VB, bool QJL>
hipError_t launch_split_q(const AttnArgs& a, hipStream_t s) {
    if (a.kc.norm_blocks == 2 || a.vc.norm_blocks == 2) {
        // two norm blocks: d = 256, no QJL, at most 8 rows per block (the plan's G)
        if constexpr (D == 256 && !QJL) {
            if (a.heads_per_chunk == 8) launch_split_g<D, KB, VB, QJL, 8, true>(a, s);
            else launch_split_g<D, KB, VB, QJL, 0, true>(a, s);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.heads_per_chunk > 8) {
        if constexpr (split_rows16(D, QJL)) launch_split_g<D, KB, VB, QJL, 16, false>(a, s);
        else return hipErrorInvalidValue;  // the plan gives such chunks only where they exist
    } else if (a.heads_per_chunk == 8) {
        launch_split_g<D, KB, VB, QJL, 8, false>(a, s);
    } else {
        launch_split_g<D, KB, VB, QJL, 0, false>(a, s);
    }
    return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
    return a.kc.qjl_m > 0 ? launch_split_q<D, KB, VB, true>(a, s) : launch_split_q<D, KB, VB, false>(a, s);
}

// Resident split blocks per compute unit for one split-kernel variant (the
// switch variants use the same LDS and launch bounds).
template <int D, int KB, int VB>
int split_blocks(bool qjl) {
    int nb = 0;
    const hipError_t e =
        qjl ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, split_kernel<D, KB, VB, true, false, false, 8, false>,
                                                          64 * split_waves(D, KB, VB, true), 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, split_kernel<D, KB, VB, false, false, false, 8, false>,
                                                          64 * split_waves(D, KB, VB, false), 0);
    return e == hipSuccess && nb > 0 ? nb : 0;
}

// Value widths of the scan at d: every width at d >= 128; at d = 64 a lane
// group's V piece needs 2 to 4 bits (and the keys 2 or 4, see tq_attn.hip).
constexpr bool scan_vb_ok(int d, int vb) { return d >= 128 || vb >= 2; }

template <int D, int KB, int VB>
hipError_t launch_split_v(const AttnArgs& a, hipStream_t s) {
    if constexpr (scan_vb_ok(D, VB)) return launch_split<D, KB, VB>(a, s);
    else return hipErrorInvalidValue;
}

template <int D, int KB>
hipError_t launch_split_dk(const AttnArgs& a, hipStream_t s) {
    switch (a.vc.bits) {
        case 1: return launch_split_v<D, KB, 1>(a, s);
        case 2: return launch_split_v<D, KB, 2>(a, s);
        case 3: return launch_split_v<D, KB, 3>(a, s);
        default: return launch_split_v<D, KB, 4>(a, s);
    }
}

template <int D, int KB, int VB>
int split_blocks_v(bool qjl) {
    if constexpr (scan_vb_ok(D, VB)) return split_blocks<D, KB, VB>(qjl);
    else return 0;
}

template <int D, int KB>
int split_blocks_dk(int vb, bool qjl) {
    switch (vb) {
        case 1: return split_blocks_v<D, KB, 1>(qjl);
        case 2: return split_blocks_v<D, KB, 2>(qjl);
        case 3: return split_blocks_v<D, KB, 3>(qjl);
        default: return split_blocks_v<D, KB, 4>(qjl);
    }
}

}  // namespace attn

// One explicit specialization per (D, KB) lives in its own translation unit.
template <int D, int KB>
hipError_t launch_split_dk(const AttnArgs& a, hipStream_t s);
template <int D, int KB>
int split_blocks_dk(int vb, bool qjl);

}  // namespace tqi
