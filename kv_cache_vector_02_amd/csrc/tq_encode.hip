// Encode and decode kernels for gfx950.
//
// Encode one vector per group of LPV = d/8 lanes: 16-byte loads, float32 norm
// by a group reduction, sign flip, register/DPP Walsh-Hadamard transform,
// Lloyd-Max index by counting scaled thresholds, bit packing with the quad's
// bytes assembled into whole dwords, half norm.  The QJL variant additionally
// stages the residual r of a 32-vector tile in LDS and forms the sign bits of
// S r with a register-tiled product against S streamed through LDS.
//
// The method steps follow "TurboQuant KV 캐시 압축 for llama.cpp" (v1.7.0
// "핵심 설계 결정" item 4: internal sign flip + butterfly WHT in the encoder;
// "약간의 비하인드": 50 B per 3-bit d=128 block) and the TurboQuant PyTorch
// write-up on idea.jsleekr.com ("핵심 발견 3": bit-shift packing).
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace {

using namespace tqd;

// Index of z = w/n with the float32 thresholds t_j: idx = #{j : z > t_j}.
// The comparison uses w against t_j*n (n > 0); the codebook is symmetric with
// t_{L/2-1} = 0, so for w > 0 idx = L/2 + #{k : w > T_k} and for w <= 0
// idx = L/2 - 1 - #{k : |w| >= T_k}, over the positive scaled thresholds T_k.
// Both counts compare non-negative floats, done exactly on their bit patterns:
// a >= T  <=>  bits(a) + 1 > bits(T).
template <int BITS>
__device__ __forceinline__ uint32_t quantize(float w, const uint32_t (&T)[(1 << BITS) / 2]) {
    constexpr int HALF = (1 << BITS) / 2;
    const uint32_t wb = as_u(w);
    const bool pos = (int32_t)wb > 0;  // w > +0 (sign clear, not zero)
    const uint32_t key = (wb & 0x7FFFFFFFu) + (pos ? 0u : 1u);
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < HALF - 1; ++k) cnt += key > T[k] ? 1u : 0u;
    return pos ? (uint32_t)HALF + cnt : (uint32_t)(HALF - 1) - cnt;
}

// Write the packed codes of one vector: each lane owns BITS bytes (8 indices);
// lane j of each quad stores dword j of the quad's 4*BITS bytes.
template <int BITS>
__device__ __forceinline__ void store_codes(uint32_t* rowp, int gl, uint32_t packed, bool valid) {
    const uint32_t p0 = quad_bcast<0>(packed), p1 = quad_bcast<1>(packed);
    const uint32_t p2 = quad_bcast<2>(packed), p3 = quad_bcast<3>(packed);
    const int j = gl & 3;
    uint32_t word = 0;
    if constexpr (BITS == 4) {
        word = packed;
    } else if constexpr (BITS == 3) {
        word = j == 0 ? (p0 | (p1 << 24)) : j == 1 ? ((p1 >> 8) | (p2 << 16)) : ((p2 >> 16) | (p3 << 8));
    } else if constexpr (BITS == 2) {
        word = j == 0 ? (p0 | (p1 << 16)) : (p2 | (p3 << 16));
    } else {
        word = p0 | (p1 << 8) | (p2 << 16) | (p3 << 24);
    }
    if (valid && j < BITS) rowp[(gl >> 2) * BITS + j] = word;
}

struct VecState {
    float v[8];
    float nrm;   // threshold scale: z = w / nrm (the norm, or nu_h sqrt(2) with two norm blocks)
    float keep;  // the norm stored for the lane's block
};

// After the first transform: the second pass of the double transform (d = 64)
// and the scales of the norm blocks (two blocks at d >= 256: lane gl holds
// rotated dims [8 gl, 8 gl + 8), so the lanes below LPV/2 hold the first half).
// ss = ||x||^2 of the input.
template <int D>
__device__ __forceinline__ void finish_rotation(VecState& st, int gl, const CodecArgs& c, float ss) {
    constexpr int LPV = D / 8;
    if constexpr (D == 64) {
        if (c.rotation == TQ_ROT_DOUBLE) second_pass<LPV>(st.v, gl, c.sign_mask3);
    }
    if constexpr (D >= 256) {
        if (c.norm_blocks == 2) {
            float sh = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sh = fmaf(st.v[e], st.v[e], sh);
            sh = group_sum<LPV / 2>(sh);  // ||y_h||^2 of the lane's half
            st.keep = __builtin_amdgcn_sqrtf(sh * (1.0f / (float)D));
            st.nrm = __builtin_amdgcn_sqrtf(sh * (2.0f / (float)D));
            return;
        }
    }
    st.nrm = st.keep = __builtin_amdgcn_sqrtf(ss);
}

// Norms of one vector in its norms row (norm_blocks halves) by the lanes
// that start a block.
template <int D>
__device__ __forceinline__ void store_norms(const EncodeArgs& a, int64_t orow, int gl, const VecState& st, bool ok) {
    constexpr int LPV = D / 8;
    const int nb = D >= 256 ? a.c.norm_blocks : 1;
    const int per = LPV / nb;
    if (ok && (gl & (per - 1)) == 0) a.norms[orow * nb + gl / per] = norm_to_half(st.keep);
}

// Input elements lane gl of a group loads: those of lane fwht_src_lane(gl)
// (the order the fused transform takes), and the sign bits of D for them.
template <int D>
__device__ __forceinline__ int enc_src_lane(int gl) { return fwht_src_lane<D / 8>(gl); }

__device__ __forceinline__ uint32_t enc_sign_bits(const uint32_t* mask, int sl) {
    return (mask[sl >> 2] >> ((sl & 3) * 8)) & 0xFFu;
}

// Norm, sign flip and transform of the 8 elements a lane holds (st.v, loaded
// from lane enc_src_lane(gl)); afterwards lane gl holds elements
// [8 gl, 8 gl + 8) of H(D x).  v_sqrt_f32 (1 ulp) gives the norm: both the
// half norm and the code decisions already allow 1e-6 relative.
template <int D>
__device__ __forceinline__ void rotate(VecState& st, int gl, uint32_t sbits, const CodecArgs& c) {
    constexpr int LPV = D / 8;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(st.v[e], st.v[e], ss);
    ss = group_sum<LPV>(ss);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.v[e] = as_f(as_u(st.v[e]) ^ (((sbits >> e) & 1u) << 31));
    fwht_fused<LPV>(st.v, gl);
    finish_rotation<D>(st, gl, c, ss);
}

// The same from the raw 16-byte words of 16-bit input: the D sign flip as
// four XORs on the packed halves (flip = the per-lane masks of
// half_sign_masks), the squared norm by v_dot2_f32_f16 / v_dot2_f32_bf16
// (the products of two 16-bit values are exact in float32), then unpack.
__device__ __forceinline__ void half_sign_masks(uint32_t sbits, uint32_t (&flip)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) flip[k] = (((sbits >> (2 * k)) & 1u) << 15) | (((sbits >> (2 * k + 1)) & 1u) << 31);
}

template <int D, int DT>
__device__ __forceinline__ void rotate_raw16(Raw8<DT>& r, const uint32_t (&flip)[4], int gl, const CodecArgs& c,
                                             VecState& st) {
    static_assert(DT != 0, "16-bit input");
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    constexpr int LPV = D / 8;
    uint32_t w[4] = {r.w[0].x ^ flip[0], r.w[0].y ^ flip[1], r.w[0].z ^ flip[2], r.w[0].w ^ flip[3]};
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (DT == 1) {
            const h2_t h = __builtin_bit_cast(h2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        } else {
            const b2_t h = __builtin_bit_cast(b2_t, w[k]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
        }
    }
    r.w[0] = make_uint4(w[0], w[1], w[2], w[3]);
    unpack8<DT>(r, st.v);
    ss = group_sum<LPV>(ss);
    fwht_fused<LPV>(st.v, gl);
    finish_rotation<D>(st, gl, c, ss);
}

// Load row `row` (or zeros) from lane sl's elements, compute the norm, sign
// flip and transform.
template <int D, int DT>
__device__ __forceinline__ void load_rotate(const EncodeArgs& a, int64_t row, bool valid, int gl, int sl,
                                            uint32_t sbits, VecState& st) {
    if (valid) {
        const char* base = static_cast<const char*>(a.x) + (row * a.x_stride + sl * 8) * elem_bytes<DT>();
        load8<DT>(base, st.v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) st.v[e] = 0.0f;
    }
    rotate<D>(st, gl, sbits, a.c);
}

// Output row of input row `row` (see EncodeArgs: plain, append or prefill
// mapping); keep = false when an append position lies outside the cache.
// Row counts below 2^32 (every call that fits a device) take 32-bit division.
__device__ __forceinline__ int64_t out_row(const EncodeArgs& a, int64_t row, bool& keep) {
    keep = true;
    if (!a.pos) {
        if (a.grp_rows <= 0) return row;
        int64_t g;
        if (a.n <= 0xFFFFFFFFll) g = (uint32_t)row / (uint32_t)a.grp_rows;
        else g = row / a.grp_rows;
        return g * a.cap + a.grp_off + (row - g * a.grp_rows);
    }
    const int p = a.pos[(uint32_t)row / (uint32_t)a.seq_heads];
    keep = p >= 0 && (int64_t)p < a.cap;
    return row * a.cap + (keep ? p : 0);
}

template <int BITS>
__device__ __forceinline__ uint32_t pack_lane(const VecState& st, const CodecArgs& c, uint32_t (&idx)[8]) {
    constexpr int HALF = (1 << BITS) / 2;
    const float sc = st.nrm > 0.0f ? st.nrm : 1.0f;
    uint32_t T[HALF];
#pragma unroll
    for (int k = 0; k < HALF - 1; ++k) T[k] = as_u(c.threshold[HALF + k] * sc);
    T[HALF - 1] = 0;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        idx[e] = quantize<BITS>(st.v[e], T);
        packed |= idx[e] << (BITS * e);
    }
    return packed;
}

// The bin table of the codec's quantizer (plan_qtab on the host): entry b =
// (#thresholds below bin b, bits of the bin's threshold or +inf).  Built by
// the whole block (the threshold loop unrolled, so the thresholds stay in
// scalar registers); returns after the barrier.  The bin edges come from the
// host's reciprocal of the scale: the plan keeps every threshold 1/32 of a bin
// from an edge, far beyond that rounding.
template <int BITS>
__device__ __forceinline__ void build_qtab(const CodecArgs& c, uint2* qtab) {
    constexpr int NT = (1 << BITS) - 1;
    for (int b = threadIdx.x; b < c.qt_n; b += blockDim.x) {
        const float z0 = ((float)b - c.qt_off) * c.qt_inv_scale;
        const float z1 = ((float)b + 1.0f - c.qt_off) * c.qt_inv_scale;
        uint32_t below = 0;
        float t = INFINITY;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float tj = c.threshold[j];
            below += tj < z0 ? 1u : 0u;
            t = (tj >= z0 && tj < z1) ? tj : t;
        }
        qtab[b] = make_uint2(below, as_u(t));
    }
    __syncthreads();
}

// Packed indices of the lane's 8 values by the bin table: the count below the
// value's bin plus one compare w > t * n with the bin's threshold (the same
// float32 comparison as the threshold count, so the same indices).
template <int BITS>
__device__ __forceinline__ uint32_t pack_lane_tab(const VecState& st, const CodecArgs& c, const uint2* qtab) {
    const float sc = st.nrm > 0.0f ? st.nrm : 1.0f;
    const float sn = c.qt_scale / sc;
    const float topf = (float)(c.qt_n - 1);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float w = st.v[e];
        // bin of w / n, clamped into the table (v_med3 under IEEE min/max
        // rules: a NaN lands in bin 0)
        const float u = __builtin_amdgcn_fmed3f(fmaf(w, sn, c.qt_off), 0.0f, topf);
        const uint2 ent = qtab[(uint32_t)u];
        const uint32_t idx = ent.x + (w > as_f(ent.y) * sc ? 1u : 0u);
        packed |= idx << (BITS * e);
    }
    return packed;
}

// Vectors per lane group per pass of the plain encoder: the loads of all of
// them go out before the first is transformed, so a wave keeps kEncBatch
// 16-byte loads per lane in flight (twice that for f32 input).  One vector's
// loads at a time left the encoder waiting on memory.
constexpr int kEncBatch = 2;

// TAB: the codec has a bin table (qt_n > 0), else the thresholds are counted.
template <int D, int BITS, int DT, bool TAB>
__device__ __forceinline__ void encode_rows(const EncodeArgs& a, const uint2* qtab, int64_t block, int64_t nblocks) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    constexpr int U = kEncBatch;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (LPV - 1), sl = enc_src_lane<D>(gl);
    const uint32_t sbits = enc_sign_bits(a.c.sign_mask, sl);
    uint32_t flip[4];
    half_sign_masks(sbits, flip);
    const int64_t wave = (block * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (nblocks * blockDim.x) >> 6;
    for (int64_t base = wave * VPW * U; base < a.n; base += nwaves * VPW * U) {
        Raw8<DT> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // rows past the end re-read the last row (never stored)
            int64_t row = base + u * VPW + lane / LPV;
            row = row < a.n ? row : a.n - 1;
            ld_stream8<DT>(static_cast<const char*>(a.x) + (row * a.x_stride + sl * 8) * elem_bytes<DT>(), raw[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * VPW + lane / LPV;
            const bool valid = row < a.n;
            VecState st;
            if constexpr (DT == 0) {
                unpack8<DT>(raw[u], st.v);
                rotate<D>(st, gl, sbits, a.c);
            } else {
                rotate_raw16<D, DT>(raw[u], flip, gl, a.c, st);
            }
            uint32_t packed;
            if constexpr (TAB) {
                packed = pack_lane_tab<BITS>(st, a.c, qtab);
            } else {
                uint32_t idx[8];
                packed = pack_lane<BITS>(st, a.c, idx);
            }
            bool keep = true;
            const int64_t orow = valid ? out_row(a, row, keep) : 0;
            uint32_t* rowp = reinterpret_cast<uint32_t*>(a.codes + orow * a.code_stride);
            store_codes<BITS>(rowp, gl, packed, valid && keep);
            store_norms<D>(a, orow, gl, st, valid && keep);
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit input with the transform on the matrix cores (d = 128 and 256, the
// plain transform; one norm, or two at d = 256): y = H D x is a dense contraction of each vector
// with the +-1 matrix H, exact in its products for fp16 and bf16 input, so a
// wave runs it as v_mfma_f32_16x16x32_{f16,bf16} with its 16 vectors as the
// 16 columns.
//   * Loads: lane l (vector n = l % 16, quarter q = l / 16) reads dims
//     32 s + 8 q .. + 7 of its vector for K step s: the B operand of step s
//     as it comes from memory; the D sign flip is an XOR on the halves.
//   * A operands: H[16 r + m][32 s + k] = (-1)^popcount((16 r + m) & (32 s + k)),
//     and with m < 16, k < 32 the exponent splits into popcount(m & k & 15),
//     (r & 1) * (k >> 4) and popcount((r >> 1) & s).  For the lane holding
//     A row m, k = 8 (l / 16) + e, so one base operand, its copy signed by
//     (-1)^(l / 32) (odd r), and the negations of both (the uniform sign
//     of (r >> 1) & s) cover every (r, s): 4 registers sets instead of
//     D/16 x D/32.
//   * Output: lane l holds y[16 r + 4 q + j] of vector n (D layout), which the
//     bin-table quantizer codes in place; 4 codes per r make one piece of
//     4 BITS bits.  The pieces go through the wave's LDS area and come back as
//     dims [D/4 q, D/4 (q + 1)) per lane, which for 2 and 4 bits are already
//     the packed code words.
// Fewer vector instructions per vector than the register transform (two
// matrix-core ops per vector at d = 128 replace 56 lane adds and DPP moves).
// ---------------------------------------------------------------------------
typedef float sf4_t __attribute__((ext_vector_type(4)));
typedef _Float16 mc_h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 mc_b2_t __attribute__((ext_vector_type(2)));

template <int DT>
struct McTypes;
template <>
struct McTypes<1> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static constexpr uint32_t one = 0x3C00u;  // 1.0 as fp16
    static __device__ __forceinline__ sf4_t mfma(v8 a, v8 b, sf4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <>
struct McTypes<2> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static constexpr uint32_t one = 0x3F80u;  // 1.0 as bf16
    static __device__ __forceinline__ sf4_t mfma(v8 a, v8 b, sf4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

constexpr int kMcVectors = 16;  // vectors per wave pass (one MFMA column each)
// staged piece bytes (1 for BITS <= 2, else 2) and the padded row of a vector
constexpr int mc_piece_bytes(int bits) { return bits <= 2 ? 1 : 2; }
constexpr int mc_row_bytes(int d, int bits) { return d / 4 * mc_piece_bytes(bits) + 16; }
constexpr int mc_stage_dw(int d, int bits) { return kMcVectors * mc_row_bytes(d, bits) / 4; }

template <int D, int BITS, int DT>
__device__ __forceinline__ void encode_rows_mc(const EncodeArgs& a, const uint2* qtab, uint32_t* stage_all,
                                               int64_t block, int64_t nblocks) {
    static_assert(D == 128 || D == 256, "matrix-core transform at d = 128 and 256");
    static_assert(DT == 1 || DT == 2, "16-bit input");
    using T = McTypes<DT>;
    typedef typename T::v8 v8;
    constexpr int NS = D / 32;                   // K steps
    constexpr int NR = D / 16;                   // output row blocks
    constexpr int PB = mc_piece_bytes(BITS);     // staged bytes per piece (4 codes)
    constexpr int RB = mc_row_bytes(D, BITS);    // staged row of one vector
    constexpr int QP = D / 16;                   // pieces per lane after the exchange
    constexpr int QW = D / 4 * BITS / 32;        // code dwords per lane
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    uint8_t* stage = reinterpret_cast<uint8_t*>(stage_all + (threadIdx.x >> 6) * mc_stage_dw(D, BITS));

    // A operands (see above): base[e] = (-1)^popcount(m & (8 (q & 1) + e)) for
    // A row m = n; the odd-r copy is signed by (-1)^(q >> 1)
    uint32_t ae[4], ao[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t w = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 8 * (q & 1) + 2 * e2 + h;
            const uint32_t neg = (uint32_t)(__builtin_popcount(n & k) & 1);
            w |= (T::one | (neg << 15)) << (16 * h);
        }
        ae[e2] = w;
        ao[e2] = w ^ ((q >> 1) ? 0x80008000u : 0u);
    }
    const v8 A[4] = {__builtin_bit_cast(v8, make_uint4(ae[0], ae[1], ae[2], ae[3])),
                     __builtin_bit_cast(v8, make_uint4(ae[0] ^ 0x80008000u, ae[1] ^ 0x80008000u,
                                                       ae[2] ^ 0x80008000u, ae[3] ^ 0x80008000u)),
                     __builtin_bit_cast(v8, make_uint4(ao[0], ao[1], ao[2], ao[3])),
                     __builtin_bit_cast(v8, make_uint4(ao[0] ^ 0x80008000u, ao[1] ^ 0x80008000u,
                                                       ao[2] ^ 0x80008000u, ao[3] ^ 0x80008000u))};
    // the D sign flip of this lane's dims 32 s + 8 q .. + 7, per step
    uint32_t flip[NS][4];
#pragma unroll
    for (int st = 0; st < NS; ++st) half_sign_masks((a.c.sign_mask[st] >> (8 * q)) & 0xFFu, flip[st]);
    const int64_t wave = (block * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (nblocks * blockDim.x) >> 6;
    // the 16-byte pieces of this lane for the pass at `base` (rows past the
    // end re-read the last one and are never stored)
    auto load = [&](int64_t base, uint4 (&x)[NS]) __attribute__((always_inline)) {
        int64_t rl = base + n;
        rl = rl < a.n ? rl : a.n - 1;
        const char* src = static_cast<const char*>(a.x) + (rl * a.x_stride + 8 * q) * 2;
#pragma unroll
        for (int st = 0; st < NS; ++st) x[st] = ld_stream4(src + 64 * st);
    };
    uint4 x[NS];
    if (wave * kMcVectors < a.n) load(wave * kMcVectors, x);
    for (int64_t base = wave * kMcVectors; base < a.n; base += nwaves * kMcVectors) {
        const int64_t row = base + n;
        const bool valid = row < a.n;
        // the next pass's loads go out before this pass's work
        uint4 xn[NS];
        const int64_t next = base + nwaves * kMcVectors;
        if (next < a.n) load(next, xn);
        float ss = 0.0f;
        sf4_t acc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = sf4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const uint32_t w[4] = {x[st].x ^ flip[st][0], x[st].y ^ flip[st][1], x[st].z ^ flip[st][2],
                                   x[st].w ^ flip[st][3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (DT == 1) {
                    const mc_h2_t h = __builtin_bit_cast(mc_h2_t, w[k]);
                    ss = __builtin_amdgcn_fdot2(h, h, ss, false);
                } else {
                    const mc_b2_t h = __builtin_bit_cast(mc_b2_t, w[k]);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
                }
            }
            const v8 b = __builtin_bit_cast(v8, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int ai = 2 * (r & 1) + (__builtin_popcount((r >> 1) & st) & 1);
                acc[r] = T::mfma(A[ai], b, acc[r]);
            }
        }
        // ||x||^2 of vector n: its four quarters are lanes n + 16 q
        ss += xor_lane<16>(ss);
        ss += xor_lane<32>(ss);
        bool keep = true;
        const int64_t orow = valid ? out_row(a, row, keep) : 0;
        // the threshold scale of each half of y (rows r < NR/2 and r >= NR/2)
        // and the norms stored: one norm, ||x||, or with two norm blocks
        // (d = 256) per half h the stored sqrt(||y_h||^2 / d) and the scale
        // sqrt(2 ||y_h||^2 / d)
        float scl[2];
        if (D == 256 && a.c.norm_blocks == 2) {
            float sh[2] = {0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) sh[r / (NR / 2)] = fmaf(acc[r][j], acc[r][j], sh[r / (NR / 2)]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                sh[h] += xor_lane<16>(sh[h]);
                sh[h] += xor_lane<32>(sh[h]);
                scl[h] = __builtin_amdgcn_sqrtf(sh[h] * (2.0f / (float)D));
            }
            if (q < 2 && valid && keep) a.norms[orow * 2 + q] = norm_to_half(__builtin_amdgcn_sqrtf(sh[q] * (1.0f / (float)D)));
        } else {
            scl[0] = scl[1] = __builtin_amdgcn_sqrtf(ss);
            if (q == 0 && valid && keep) a.norms[orow] = norm_to_half(scl[0]);
        }
        // codes of y[16 r + 4 q + j], one piece of 4 codes per r, staged.  The
        // bin coordinate takes 1/sc by v_rcp_f32 (1 ulp): it only picks the
        // table bin, and every threshold lies 1/32 of a bin from a bin edge
        float scs[2], sns[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            scs[h] = scl[h] > 0.0f ? scl[h] : 1.0f;
            sns[h] = a.c.qt_scale * __builtin_amdgcn_rcpf(scs[h]);
        }
        const float topf = (float)(a.c.qt_n - 1);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float sc = scs[r / (NR / 2)], sn = sns[r / (NR / 2)];
            uint32_t piece = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = acc[r][j];
                const float u = __builtin_amdgcn_fmed3f(fmaf(w, sn, a.c.qt_off), 0.0f, topf);
                const uint2 ent = qtab[(uint32_t)u];
                const uint32_t idx = ent.x + (w > as_f(ent.y) * sc ? 1u : 0u);
                piece |= idx << (BITS * j);
            }
            uint8_t* dst = stage + n * RB + (4 * r + q) * PB;
            if constexpr (PB == 1) *dst = (uint8_t)piece;
            else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)piece;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // pieces QP q .. QP q + QP - 1 of vector n: its dims [D/4 q, D/4 (q + 1))
        const uint8_t* srcp = stage + n * RB + QP * q * PB;
        uint32_t cw[QW];
        if constexpr (BITS == 4 || BITS == 2) {
            // pieces of 16 (8) bits side by side are the packed code words
#pragma unroll
            for (int i = 0; i < QW; i += 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(srcp + 4 * i);
                cw[i] = v.x;
                cw[i + 1] = v.y;
            }
        } else {
            // 4-bit pieces in bytes (1 bit) or 12-bit pieces in halfwords (3 bits)
            constexpr int PBITS = 4 * BITS;
#pragma unroll
            for (int i = 0; i < QW; ++i) cw[i] = 0u;
#pragma unroll
            for (int p = 0; p < QP; ++p) {
                const uint32_t v = PB == 1 ? (uint32_t)srcp[p] : (uint32_t)reinterpret_cast<const uint16_t*>(srcp)[p];
                const int bit = PBITS * p;
                cw[bit >> 5] |= v << (bit & 31);
                if ((bit & 31) + PBITS > 32) cw[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (valid && keep) {
            uint32_t* rowp = reinterpret_cast<uint32_t*>(a.codes + orow * a.code_stride) + QW * q;
#pragma unroll
            for (int i = 0; i < QW; ++i) rowp[i] = cw[i];
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) x[st] = xn[st];
    }
}

// MC: the matrix-core transform (encode_rows_mc; 16-bit input, d = 128 or 256,
// the plain transform, a bin table), else the register transform.
template <int D, int BITS, int DT, bool TAB, bool MC>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
    __shared__ uint2 qtab[TAB ? kQTabMax : 1];
    __shared__ uint32_t stage[MC ? 4 * mc_stage_dw(D, BITS) : 1];
    if constexpr (TAB) build_qtab<BITS>(a.c, qtab);
    if constexpr (MC) encode_rows_mc<D, BITS, DT>(a, qtab, stage, blockIdx.x, gridDim.x);
    else encode_rows<D, BITS, DT, TAB>(a, qtab, blockIdx.x, gridDim.x);
}

// Two encodes in one launch (a layer's K and V): blocks [0, kblocks) run job
// k, the rest job v; each block switches on its codec's bit width (uniform
// per block).  Neither job uses QJL.
template <int D, int DT, bool TAB, bool MC>
__global__ __launch_bounds__(256) void encode_pair_kernel(EncodeArgs k, EncodeArgs v, int kblocks) {
    // each branch reads its own argument directly (selecting a reference to
    // one of the two would copy them to scratch)
    __shared__ uint2 qtab[TAB ? kQTabMax : 1];
    __shared__ uint32_t stage[MC ? 4 * mc_stage_dw(D, 4) : 1];  // 4 bits need the most
    auto run = [&](const EncodeArgs& a, int64_t block, int64_t nblocks) __attribute__((always_inline)) {
        auto one = [&](auto bc) __attribute__((always_inline)) {
            constexpr int B = decltype(bc)::value;
            if constexpr (TAB) build_qtab<B>(a.c, qtab);
            if constexpr (MC) encode_rows_mc<D, B, DT>(a, qtab, stage, block, nblocks);
            else encode_rows<D, B, DT, TAB>(a, qtab, block, nblocks);
        };
        switch (a.c.bits) {
            case 1: one(std::integral_constant<int, 1>{}); break;
            case 2: one(std::integral_constant<int, 2>{}); break;
            case 3: one(std::integral_constant<int, 3>{}); break;
            default: one(std::integral_constant<int, 4>{}); break;
        }
    };
    if ((int)blockIdx.x < kblocks) run(k, blockIdx.x, kblocks);
    else run(v, (int64_t)blockIdx.x - kblocks, (int64_t)gridDim.x - kblocks);
}

// QJL variant: a block of 256 threads encodes a tile of 64 vectors.
constexpr int QJL_TILE = 64;

typedef _Float16 sh8v_t __attribute__((ext_vector_type(8)));
typedef float sf4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sh8v_t as_sh8v(uint4 u) { return __builtin_bit_cast(sh8v_t, u); }
__device__ __forceinline__ uint32_t pack_h2f(float a, float b) {
    const _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D, int BITS, int DT>
__global__ __launch_bounds__(256) void encode_qjl_kernel(EncodeArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    constexpr int RS = D + 1;  // padded row of r in LDS
    constexpr int KS = D / 16;  // projection k steps (16 dims each)
    // the tile's residuals r (phase 1), then, once every wave holds its
    // operands, the S operands of two projection blocks (double buffer:
    // [block][ks][lane])
    constexpr int R_U4 = (QJL_TILE * RS + 3) / 4, SA_U4 = 2 * KS * 64;
    __shared__ __attribute__((aligned(16))) uint4 qarea[R_U4 > SA_U4 ? R_U4 : SA_U4];
    float* r_lds = reinterpret_cast<float*>(qarea);
    uint4* sa = qarea;
    __shared__ float cent[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int gl = lane & (LPV - 1), sl = enc_src_lane<D>(gl);
    const uint32_t sbits = enc_sign_bits(a.c.sign_mask, sl);
    const int m = a.c.qjl_m;
    const float rsd = 1.0f / sqrtf((float)D);
    if (tid < 16) cent[tid] = a.c.centroid[tid];
    __syncthreads();

    for (int64_t tile0 = (int64_t)blockIdx.x * QJL_TILE; tile0 < a.n; tile0 += (int64_t)gridDim.x * QJL_TILE) {
        // phase 1: codes, norm, residual -> LDS, gamma
        for (int vb = wave * VPW; vb < QJL_TILE; vb += 4 * VPW) {
            const int vloc = vb + lane / LPV;
            const int64_t row = tile0 + vloc;
            const bool valid = row < a.n;
            VecState st;
            load_rotate<D, DT>(a, row, valid, gl, sl, sbits, st);
            uint32_t idx[8];
            const uint32_t packed = pack_lane<BITS>(st, a.c, idx);
            bool keep = true;
            const int64_t orow = valid ? out_row(a, row, keep) : 0;
            uint32_t* rowp = reinterpret_cast<uint32_t*>(a.codes + orow * a.code_stride);
            store_codes<BITS>(rowp, gl, packed, valid && keep);
            const float inv = st.nrm > 0.0f ? 1.0f / st.nrm : 0.0f;
            float g2 = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float z = st.v[e] * inv;
                const float r = (z - cent[idx[e]]) * rsd;
                r_lds[vloc * RS + gl * 8 + e] = r;
                g2 = fmaf(r, r, g2);
            }
            g2 = group_sum<LPV>(g2);
            if (valid && keep && gl == 0) {
                a.norms[orow] = norm_to_half(st.nrm);
                a.gamma[orow] = norm_to_half(sqrtf(g2));
            }
        }
        __syncthreads();
        // phase 2: U = R S^T on the matrix cores (v_mfma_f32_16x16x32_f16), 16
        // projections x 8 vectors per step with the hi/lo fold of the decode
        // scan: lane (n, grp) holds in its k slots dims 16 ks + 4 grp + [0, 4)
        // as (s_hi, s_hi, s_lo, s_lo) pairs of projection 16 jb + n (A), and
        // columns 0-7 / 8-15 hold r_hi / r_lo of 8 vectors (B, zero on the
        // s_lo slots); D[j][v] + D[j][v + 8] is (S r)_j without the s_lo r_lo
        // term (below 2^-21 of the sum of |s_i r_i|).  S is scaled by 16 and r
        // by 2^15 (|r_i| < 1), so every lo part is a normal half; the signs do
        // not depend on the scale.  A wave takes 16 vectors as two column sets,
        // so each S operand read from LDS feeds two steps.  The projection
        // blocks' S operands are built once per block into LDS, the next
        // block's while this one's run.
        const int n = lane & 15, grp = lane >> 4;
        const bool lo_col = n >= 8;
        sh8v_t bq[2][KS];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int vv = 16 * wave + 8 * c + (n & 7);  // column set c's vector of the tile
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = r_lds[vv * RS + 16 * ks + 4 * grp + i] * 32768.0f;
                    const float h = (float)(_Float16)v;
                    x[i] = lo_col ? v - h : h;
                }
                bq[c][ks] = lo_col ? as_sh8v(make_uint4(pack_h2f(x[0], x[1]), 0u, pack_h2f(x[2], x[3]), 0u))
                                   : as_sh8v(make_uint4(pack_h2f(x[0], x[1]), pack_h2f(x[0], x[1]),
                                                        pack_h2f(x[2], x[3]), pack_h2f(x[2], x[3])));
            }
        }
        __syncthreads();  // every wave holds its operands: r's space takes the S operands
        constexpr int NE = KS * 64;              // S operands of one projection block
        constexpr int BPT = (NE + 255) / 256;    // ... each thread builds
        const int jbs = m >> 4;             // projection blocks
        float4 sv[BPT];
        auto s_load = [&](int jb) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < BPT; ++u) {
                const int e = tid + 256 * u, ks = e >> 6, l = e & 63;
                if (NE % 256 == 0 || e < NE)
                    sv[u] = *reinterpret_cast<const float4*>(a.S + (int64_t)(16 * jb + (l & 15)) * D + 16 * ks +
                                                             4 * (l >> 4));
            }
        };
        auto s_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < BPT; ++u) {
                if (!(NE % 256 == 0 || tid + 256 * u < NE)) continue;
                const float x[4] = {16.0f * sv[u].x, 16.0f * sv[u].y, 16.0f * sv[u].z, 16.0f * sv[u].w};
                float h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = (float)(_Float16)x[i];
                sa[buf * KS * 64 + tid + 256 * u] = make_uint4(pack_h2f(h[0], h[1]), pack_h2f(x[0] - h[0], x[1] - h[1]),
                                                               pack_h2f(h[2], h[3]), pack_h2f(x[2] - h[2], x[3] - h[3]));
            }
        };
        // the output rows of this lane's two vectors (lanes n < 8 of lane
        // group 0 write their vectors' signs)
        bool writer[2];
        uint32_t* qrow[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bool keep = true;
            const int64_t vrow = tile0 + 16 * wave + 8 * c + (n & 7);
            const int64_t orow = vrow < a.n ? out_row(a, vrow, keep) : 0;
            writer[c] = n < 8 && grp == 0 && vrow < a.n && keep;
            qrow[c] = reinterpret_cast<uint32_t*>(a.qjl + orow * (m >> 3));
        }
        s_load(0);
        s_store(0);
        __syncthreads();
        uint32_t word[2] = {0u, 0u};
        for (int jb = 0; jb < jbs; ++jb) {
            const int cur = jb & 1;
            if (jb + 1 < jbs) s_load(jb + 1);  // uniform; the loads run under the matrix-core steps
            const uint4* sc = sa + cur * KS * 64 + lane;
            sf4v_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const sh8v_t sop = as_sh8v(sc[ks * 64]);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sop, bq[0][ks], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sop, bq[1][ks], acc[1], 0, 0, 0);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // lanes n < 8: projections 16 jb + 4 grp + i of the set's vector; bit = [u >= 0]
                uint32_t f = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) f |= ((acc[c][i] + xor_lane<8>(acc[c][i])) >= 0.0f ? 1u : 0u) << i;
                f |= xor_lane_u<16>(f) << 4;  // lane group 0 gathers the 16 projections
                f |= xor_lane_u<32>(f) << 8;
                word[c] |= (f & 0xFFFFu) << (16 * (jb & 1));
                if (jb & 1) {
                    if (writer[c]) qrow[c][jb >> 1] = word[c];
                    word[c] = 0;
                }
            }
            if (jb + 1 < jbs) s_store(cur ^ 1);
            __syncthreads();  // the next block's operands are in; this block's are free
        }
    }
}

// Residual signs without a dense projection (one vector per lane group, in
// registers): the structured SRHT QJL, bits = signs of H(D2 r) with the second
// sign basis D2 and gamma = ||r|| ("TurboQuant KV 캐시 압축 for llama.cpp",
// v1.3.0 and v1.4.2 item 2: the paper's QJL is SRHT-based, with its own signs2),
// or Direct Sign, bits = signs of r with gamma = mean |r_i| (v1.1.0 "Direct
// Sign").  r = (z - c[idx]) / sqrt(d) as for the Gaussian QJL.
template <int D, int BITS, int DT, int KIND>
__global__ __launch_bounds__(256) void encode_sign_kernel(EncodeArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    __shared__ float cent[16];
    if (threadIdx.x < 16) cent[threadIdx.x] = a.c.centroid[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int gl = lane & (LPV - 1), sl = enc_src_lane<D>(gl);
    const uint32_t sbits = enc_sign_bits(a.c.sign_mask, sl);
    const uint32_t sbits2 = (a.c.sign_mask2[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
    const float rsd = 1.0f / sqrtf((float)D);
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t base = wave * VPW; base < a.n; base += nwaves * VPW) {
        const int64_t row = base + lane / LPV;
        const bool valid = row < a.n;
        VecState st;
        load_rotate<D, DT>(a, row, valid, gl, sl, sbits, st);
        uint32_t idx[8];
        const uint32_t packed = pack_lane<BITS>(st, a.c, idx);
        bool keep = true;
        const int64_t orow = valid ? out_row(a, row, keep) : 0;
        store_codes<BITS>(reinterpret_cast<uint32_t*>(a.codes + orow * a.code_stride), gl, packed, valid && keep);
        const float inv = st.nrm > 0.0f ? 1.0f / st.nrm : 0.0f;
        float r[8], acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            r[e] = (st.v[e] * inv - cent[idx[e]]) * rsd;
            acc += KIND == TQ_RES_SIGN ? fabsf(r[e]) : r[e] * r[e];
        }
        acc = group_sum<LPV>(acc);
        const float gamma = KIND == TQ_RES_SIGN ? acc * (1.0f / (float)D) : sqrtf(acc);
        if constexpr (KIND == TQ_RES_SRHT) {
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = as_f(as_u(r[e]) ^ (((sbits2 >> e) & 1u) << 31));
            fwht<LPV>(r, gl);
        }
        uint32_t sb = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb |= (r[e] >= 0.0f ? 1u : 0u) << e;
        store_codes<1>(reinterpret_cast<uint32_t*>(a.qjl + orow * (D / 8)), gl, sb, valid && keep);
        if (valid && keep && gl == 0) {
            a.norms[orow] = norm_to_half(st.nrm);
            a.gamma[orow] = norm_to_half(gamma);
        }
    }
}

template <int D, int BITS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    __shared__ float cent[16];
    if (threadIdx.x < 16) cent[threadIdx.x] = a.c.centroid[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int gl = lane & (LPV - 1);
    const uint32_t sbits = (a.c.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
    const int nb = D >= 256 ? a.c.norm_blocks : 1;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t base = wave * VPW; base < a.n; base += nwaves * VPW) {
        const int64_t row = base + lane / LPV;
        const bool valid = row < a.n;
        const int64_t r = valid ? row : 0;
        const uint8_t* rp = a.codes + r * a.code_stride + gl * BITS;
        uint32_t packed = 0;
#pragma unroll
        for (int k = 0; k < BITS; ++k) packed |= (uint32_t)rp[k] << (8 * k);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = cent[(packed >> (BITS * e)) & ((1u << BITS) - 1u)];
        // x_hat = D R(y_hat) / d with y_hat = n c (one norm) or nu_h sqrt(2) c on
        // block h (two norms); R = H, or H D3 H / sqrt(d) (the same pass after H)
        float sc;
        if (nb == 2) {
            const float nu = half_bits_to_float(a.norms[r * 2 + (gl >= LPV / 2 ? 1 : 0)]);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= nu * 1.41421356237309505f;
            sc = 1.0f / (float)D;
        } else {
            sc = half_bits_to_float(a.norms[r]) * (1.0f / (float)D);
        }
        fwht<LPV>(v, gl);
        if constexpr (D == 64) {
            if (a.c.rotation == TQ_ROT_DOUBLE) second_pass<LPV>(v, gl, a.c.sign_mask3);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e] * sc) ^ (((sbits >> e) & 1u) << 31));
        if (valid) {
            float4* o = reinterpret_cast<float4*>(a.out + row * D + gl * 8);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

// Blocks of the plain encoder for n rows at d: 4 waves, each taking
// kEncBatch * 64/(d/8) rows per pass; at most 4096 blocks (16 per compute
// unit), the rows loop inside.
int encode_blocks(int64_t n, int d) {
    const int64_t vpb = 4 * kEncBatch * (64 / (d / 8));
    const int64_t need = (n + vpb - 1) / vpb;
    return (int)(need < 4096 ? need : 4096);
}

// The matrix-core encoder: shapes it is built for, codecs it serves, and its
// blocks (4 waves of 16 vectors per pass, at most 4096 blocks).
constexpr bool mc_dims(int d, int dt) { return (d == 128 || d == 256) && dt != 0; }
bool mc_codec(const CodecArgs& c) {
    return c.rotation == TQ_ROT_WHT && (c.norm_blocks == 1 || c.d == 256) && c.qt_n > 0;
}
// One resident round of blocks (compute units x resident blocks of the
// kernel, cached per kernel): each wave then loops over several passes and
// its next pass's loads overlap this pass's work.
template <auto Kernel>
int mc_blocks(int64_t n) {
    static std::atomic<int> per_cu{0};
    int pc = per_cu.load(std::memory_order_relaxed);
    if (pc <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, Kernel, 256, 0) != hipSuccess || pc <= 0) pc = 4;
        per_cu.store(pc, std::memory_order_relaxed);
    }
    const int64_t need = (n + 4 * kMcVectors - 1) / (4 * kMcVectors);
    const int64_t cap = (int64_t)device_cus() * pc;
    return (int)(need < cap ? need : cap);
}

template <int D, int BITS, int DT>
hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t s) {
    if constexpr (D > 256) {
        // d = 512 codecs have no residual (checked on the host)
    } else if (a.c.residual == TQ_RES_SRHT || a.c.residual == TQ_RES_SIGN) {
        constexpr int VPB = 4 * (64 / (D / 8));
        const int64_t need = (a.n + VPB - 1) / VPB;
        const int grid = (int)(need < 16384 ? need : 16384);
        if (a.c.residual == TQ_RES_SRHT)
            hipLaunchKernelGGL((encode_sign_kernel<D, BITS, DT, TQ_RES_SRHT>), dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((encode_sign_kernel<D, BITS, DT, TQ_RES_SIGN>), dim3(grid), dim3(256), 0, s, a);
    } else if (a.c.qjl_m > 0) {
        const int64_t tiles = (a.n + QJL_TILE - 1) / QJL_TILE;
        const int grid = (int)(tiles < 8192 ? tiles : 8192);
        hipLaunchKernelGGL((encode_qjl_kernel<D, BITS, DT>), dim3(grid), dim3(256), 0, s, a);
    }
    if (a.c.qjl_m == 0) {
        if constexpr (mc_dims(D, DT)) {
            if (mc_codec(a.c)) {
                constexpr auto kern = encode_kernel<D, BITS, DT, true, true>;
                hipLaunchKernelGGL(kern, dim3(mc_blocks<kern>(a.n)), dim3(256), 0, s, a);
                return hipGetLastError();
            }
        }
        if (a.c.qt_n > 0)
            hipLaunchKernelGGL((encode_kernel<D, BITS, DT, true, false>), dim3(encode_blocks(a.n, D)), dim3(256), 0, s,
                               a);
        else
            hipLaunchKernelGGL((encode_kernel<D, BITS, DT, false, false>), dim3(encode_blocks(a.n, D)), dim3(256), 0,
                               s, a);
    }
    return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_encode_b(const EncodeArgs& a, hipStream_t s) {
    switch (a.c.bits) {
        case 1: return launch_encode_t<D, 1, DT>(a, s);
        case 2: return launch_encode_t<D, 2, DT>(a, s);
        case 3: return launch_encode_t<D, 3, DT>(a, s);
        default: return launch_encode_t<D, 4, DT>(a, s);
    }
}

template <int DT>
hipError_t launch_encode_d(const EncodeArgs& a, hipStream_t s) {
    switch (a.c.d) {
        case 32: return launch_encode_b<32, DT>(a, s);
        case 64: return launch_encode_b<64, DT>(a, s);
        case 128: return launch_encode_b<128, DT>(a, s);
        case 256: return launch_encode_b<256, DT>(a, s);
        default: return launch_encode_b<512, DT>(a, s);
    }
}

template <int D>
hipError_t launch_decode_b(const DecodeArgs& a, hipStream_t s) {
    constexpr int VPB = 4 * (64 / (D / 8));
    const int64_t need = (a.n + VPB - 1) / VPB;
    const int grid = (int)(need < 16384 ? need : 16384);
    switch (a.c.bits) {
        case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), dim3(grid), dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), dim3(grid), dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_kernel<D, 3>), dim3(grid), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((decode_kernel<D, 4>), dim3(grid), dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

template <int D, int DT>
static hipError_t launch_pair_d(const EncodeArgs& k, const EncodeArgs& v, hipStream_t s) {
    if constexpr (mc_dims(D, DT)) {
        if (mc_codec(k.c) && mc_codec(v.c)) {
            // the K and V jobs share one resident round in proportion to their rows
            constexpr auto kern = encode_pair_kernel<D, DT, true, true>;
            int all = mc_blocks<kern>(k.n + v.n);
            all = all < 2 ? 2 : all;
            int kb = (int)((int64_t)all * k.n / (k.n + v.n));
            kb = kb < 1 ? 1 : (kb > all - 1 ? all - 1 : kb);  // each job gets at least one block
            hipLaunchKernelGGL(kern, dim3(all), dim3(256), 0, s, k, v, kb);
            return hipGetLastError();
        }
    }
    const int kb = encode_blocks(k.n, D), vb = encode_blocks(v.n, D);
    if (k.c.qt_n > 0 && v.c.qt_n > 0)
        hipLaunchKernelGGL((encode_pair_kernel<D, DT, true, false>), dim3(kb + vb), dim3(256), 0, s, k, v, kb);
    else
        hipLaunchKernelGGL((encode_pair_kernel<D, DT, false, false>), dim3(kb + vb), dim3(256), 0, s, k, v, kb);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_pair_t(const EncodeArgs& k, const EncodeArgs& v, hipStream_t s) {
    switch (k.c.d) {
        case 32: return launch_pair_d<32, DT>(k, v, s);
        case 64: return launch_pair_d<64, DT>(k, v, s);
        case 128: return launch_pair_d<128, DT>(k, v, s);
        case 256: return launch_pair_d<256, DT>(k, v, s);
        default: return launch_pair_d<512, DT>(k, v, s);
    }
}

hipError_t launch_encode_pair(const EncodeArgs& k, const EncodeArgs& v, int dtype, hipStream_t s) {
    // a QJL key codec keeps its own kernel: two launches then
    if (k.c.qjl_m > 0 || v.c.qjl_m > 0 || k.n == 0 || v.n == 0) {
        hipError_t e = k.n > 0 ? launch_encode(k, dtype, s) : hipSuccess;
        if (e == hipSuccess && v.n > 0) e = launch_encode(v, dtype, s);
        return e;
    }
    switch (dtype) {
        case TQ_F32: return launch_pair_t<0>(k, v, s);
        case TQ_F16: return launch_pair_t<1>(k, v, s);
        default: return launch_pair_t<2>(k, v, s);
    }
}

hipError_t launch_encode(const EncodeArgs& a, int dtype, hipStream_t s) {
    switch (dtype) {
        case TQ_F32: return launch_encode_d<0>(a, s);
        case TQ_F16: return launch_encode_d<1>(a, s);
        default: return launch_encode_d<2>(a, s);
    }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    switch (a.c.d) {
        case 32: return launch_decode_b<32>(a, s);
        case 64: return launch_decode_b<64>(a, s);
        case 128: return launch_decode_b<128>(a, s);
        case 256: return launch_decode_b<256>(a, s);
        default: return launch_decode_b<512>(a, s);
    }
}

}  // namespace tqi
