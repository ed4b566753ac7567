// Decode attention over head dimension 512 on the matrix cores, with one norm
// per vector or one per half of the rotated vector ("TurboQuant KV 캐시 압축
// for llama.cpp", v1.5.2 "핵심 변경" item 5; v1.5.0 and v1.5.1 for the 512-point
// transform).
//
// Grid (splits, kv head x head chunk, batch); a block of 4 waves takes its
// split's 64-token tiles one after the other, every wave on the same tile and
// each wave on its own quarter of the 512 dims.  A quarter lies inside one norm
// half, so per-half norms need no split of a matrix-core sum.  Per tile:
//   * partial scores of the wave's quarter, v_mfma_f32_16x16x32_f16 with the
//     scan's hi/lo fold (16 tokens x 8 heads per step: c_hi and c_lo of 4 dims
//     per lane in the k slots, q_hi in columns 0-7 and q_lo in 8-15), scaled
//     by the token's norm of that half and written to LDS;
//   * one block barrier; every wave then sums the four partials of the tokens
//     it needs and runs the same online softmax (the waves agree bit for bit);
//   * value sums of the wave's quarter: weights p |v| (half) as the A operand
//     (head rows, token k slots), centroid halves as B (column n' of N block nb
//     stands for dim 8 n' + nb, so a lane's codes of one token are one
//     contiguous 8-code piece of the staged row), one pair table lookup per two
//     dims and token, v_perm pairing two tokens per B dword.
// The block writes one partial (max, sum, acc[d]) per query row in the layout
// the combine kernel merges; sums stay in the rotated domain.
#include <hip/hip_runtime.h>
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace {

using namespace tqd;

typedef _Float16 mh8_t __attribute__((ext_vector_type(8)));
typedef float mf4_t __attribute__((ext_vector_type(4)));

constexpr int kMcRows = 8;     // query heads per block at most (columns 0-7)
constexpr int kPStride = 68;   // LDS floats per head row of a wave's 64 partial scores
constexpr float kLog2eMc = 1.4426950408889634f;

__device__ __forceinline__ mh8_t as_mh8(uint4 u) { return __builtin_bit_cast(mh8_t, u); }

__device__ __forceinline__ uint32_t pack_halves(float a, float b) {
    const _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// bits [bit0, bit0 + NB) of a little-endian dword array (bit0 a compile-time
// constant after unrolling)
template <int NB>
__device__ __forceinline__ uint32_t bits_from(const uint32_t* w, int bit0) {
    const int wi = bit0 >> 5, sh = bit0 & 31;
    if (sh + NB <= 32) return (w[wi] >> sh) & ((1u << NB) - 1u);
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << NB) - 1u);
}

__device__ __forceinline__ void wave_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KB, int VB>
__global__ __launch_bounds__(256) void wide_mc_kernel(AttnArgs a) {
    constexpr int D = 512;
    constexpr int DW = D / 4;           // dims of one wave
    constexpr int DG = DW / 4;          // dims of one lane group in the score layout
    constexpr int KS = DG / 4;          // score k steps
    constexpr int NB = DW / 16;         // value N blocks (8)
    constexpr int RBK = D * KB / 8, RBV = D * VB / 8;
    constexpr int SEGV = DW * VB / 8;   // bytes of a wave's value quarter of one token
    constexpr int SEGW = SEGV / 4;      // ... dwords
    constexpr int VSTR = SEGW + 1;      // padded LDS stride of the staged quarters
    constexpr int PIECE = 8 * VB;       // bits of a lane's 8 dims of one token
    constexpr int KTE = 1 << (2 * KB), KTS = KB <= 3 ? 32 : 8;  // K pair table: entries, copies
    // V pair table: one copy per lane of the wave (16 at 4 bits), so the 64
    // four-byte reads of a lookup fall on distinct banks
    constexpr int VTE = 1 << (2 * VB), VTS = VB <= 3 ? 64 : 16;
    constexpr int PB = 4 * kMcRows * kPStride;                  // floats of one partial buffer
    static_assert(NB == 8 && KS == 8 && PIECE <= 32, "layout");
    __shared__ __attribute__((aligned(16))) uint2 ktab[KTE * KTS];   // (c_hi a, c_hi b), (c_lo a, c_lo b) of 16 c
    __shared__ __attribute__((aligned(16))) uint32_t vtab[VTE * VTS];  // (c a, c b) halves
    // the rotated queries are read only before the tile loop: the loop's
    // partial scores and staged value quarters reuse their space
    constexpr int LOOP_DW = 2 * PB + 4 * 64 * VSTR;
    constexpr int AREA_DW = LOOP_DW > kMcRows * D ? LOOP_DW : kMcRows * D;
    __shared__ __attribute__((aligned(16))) uint32_t area[AREA_DW];
    float* qr = reinterpret_cast<float*>(area);
    float* psc = reinterpret_cast<float*>(area);
    uint32_t* vst = area + 2 * PB;
    __shared__ __attribute__((aligned(16))) float nrms[4 * 128];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.chunks, chunk = blockIdx.y - kvh * a.chunks;
    const int b = blockIdx.z;
    const int G = a.heads_per_chunk;
    const int cap = (int)a.ctx_cap;
    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int t_beg = split * (int)a.split_tokens;
    const int t_end = (t_beg + (int)a.split_tokens < ctx) ? t_beg + (int)a.split_tokens : ctx;
    const int64_t kvrow = ((int64_t)b * a.hkv + kvh) * a.ctx_cap;
    const int row0 = kvh * a.g + chunk * G;  // first query head of the block

    for (int i = tid; i < KTE * KTS; i += 256) {
        const int e = i / KTS;
        const float fa = 16.0f * a.kc.centroid[e & ((1 << KB) - 1)];
        const float fb = 16.0f * a.kc.centroid[e >> KB];
        const float ha = (float)(_Float16)fa, hb = (float)(_Float16)fb;
        ktab[i] = make_uint2(pack_halves(ha, hb), pack_halves(fa - ha, fb - hb));
    }
    for (int i = tid; i < VTE * VTS; i += 256) {
        const int e = i / VTS;
        vtab[i] = pack_halves(a.vc.centroid[e & ((1 << VB) - 1)], a.vc.centroid[e >> VB]);
    }
    // rotated queries qr[r][i] = (scale log2(e) / d) H(D_K q_r), rows G.. zero:
    // one 64-lane group per row
    for (int r = wave; r < kMcRows; r += 4) {
        float x[8];
        if (r < G) {
            const int64_t e0 = ((int64_t)b * a.hq + row0 + r) * D + 8 * lane;
            if (a.q_dtype == TQ_F32) load8<0>(static_cast<const float*>(a.q) + e0, x);
            else if (a.q_dtype == TQ_F16) load8<1>(static_cast<const uint16_t*>(a.q) + e0, x);
            else load8<2>(static_cast<const uint16_t*>(a.q) + e0, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
        const uint32_t sb = (a.kc.sign_mask[lane >> 2] >> ((lane & 3) * 8)) & 0xFFu;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = as_f(as_u(x[e]) ^ (((sb >> e) & 1u) << 31));
        fwht<64>(x, lane);
        const float qs = a.scale * kLog2eMc / (float)D;
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[r * D + 8 * lane + e] = x[e] * qs;
    }
    __syncthreads();

    // this wave's query operands: column n <-> head n & 7, hi (n < 8) or lo;
    // lane group grp, k step ks: dims DW wave + DG grp + 4 ks + [0, 4).  The
    // wave's quarter is scaled by one power of two into [2^14, 2^15) and the
    // centroids by 16, so every lo part is a normal half.
    const int hq = n & 7;
    const bool lo_col = n >= 8;
    mh8_t bq[KS];
    float qinv;
    {
        float amax = 0.0f;
        for (int i = lane; i < kMcRows * DW; i += 64) amax = fmaxf(amax, fabsf(qr[(i / DW) * D + DW * wave + i % DW]));
        amax = fmaxf(amax, xor_lane<1>(amax));
        amax = fmaxf(amax, xor_lane<2>(amax));
        amax = fmaxf(amax, xor_lane<4>(amax));
        amax = fmaxf(amax, xor_lane<8>(amax));
        amax = fmaxf(amax, xor_lane<16>(amax));
        amax = fmaxf(amax, xor_lane<32>(amax));
        float sc = 1.0f;
        if (amax > 0.0f && isfinite(amax)) {
            int ex;
            frexpf(amax, &ex);
            sc = ldexpf(1.0f, 15 - ex);
        }
        qinv = 1.0f / (16.0f * sc);
        const float* qrow = qr + hq * D + DW * wave + DG * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = qrow[4 * ks + i] * sc;
                const float h = (float)(_Float16)v;
                x[i] = lo_col ? v - h : h;
            }
            // slots (hi d0, hi d1, lo d0, lo d1, hi d2, hi d3, lo d2, lo d3) of the A side
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool lo_slot = (e & 2) != 0;
                bq[ks][e] = (lo_col && lo_slot) ? (_Float16)0.0f : (_Float16)x[(e >> 2) * 2 + (e & 1)];
            }
        }
    }
    __syncthreads();  // every wave has its query operands: the area is the loop's now

    const int nbk = a.kc.norm_blocks, nbv = a.vc.norm_blocks;
    const float bs_k = nbk == 2 ? 1.41421356237309505f : 1.0f;  // sqrt(B)
    const float bs_v = nbv == 2 ? 1.41421356237309505f : 1.0f;
    const int kblk = nbk == 2 ? (wave >> 1) : 0;  // norm half of this wave's dims
    const int vblk = nbv == 2 ? (wave >> 1) : 0;
    const uint16_t* kn = a.k_norms + kvrow * nbk + kblk;
    const uint16_t* vn = a.v_norms + kvrow * nbv + vblk;
    const uint8_t* kcodes = a.k_codes + kvrow * RBK;
    const uint8_t* vcodes = a.v_codes + kvrow * RBV;
    const uint2* ktl = ktab + lane % KTS;
    constexpr int VLOG = VTS == 64 ? 8 : 6;       // log2 of the V table's row stride in bytes
    const uint32_t vlane = (uint32_t)(lane % VTS) * 4u;  // this lane's copy in a row
    uint32_t* vs = vst + wave * 64 * VSTR;
    const bool live_row = n < 8 && hq < G;  // A rows of the value sums that carry a head

    mf4_t vacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vacc[nb] = mf4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f;  // of head hq

    // a tile's global inputs, requested one tile ahead: the lane's key codes of
    // tokens 16 tb + n (its lane group's 32 codes), its token's value quarter
    // and its token's norms of this wave's halves (tokens clamped to the split)
    struct TileIn {
        uint32_t cw[4][KB];
        uint4 vq[VB];
        uint32_t nk, nv;
    };
    auto fetch = [&](TileIn& in, int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int tok = t0 + 16 * tb + n;
            const int tk = tok < t_end ? tok : t_end - 1;
            const uint32_t* kp = reinterpret_cast<const uint32_t*>(kcodes + (int64_t)tk * RBK) + (4 * wave + grp) * KB;
            if constexpr (KB == 4) {
                const uint4 v = ld_stream4(kp);
                in.cw[tb][0] = v.x; in.cw[tb][1] = v.y; in.cw[tb][2] = v.z; in.cw[tb][3] = v.w;
            } else if constexpr (KB == 2) {
                const uint2 v = ld_stream2(kp);
                in.cw[tb][0] = v.x; in.cw[tb][1] = v.y;
            } else {
#pragma unroll
                for (int u = 0; u < KB; ++u) in.cw[tb][u] = ld_stream1(kp + u);
            }
        }
        const int tv = (t0 + lane < t_end) ? t0 + lane : t_end - 1;
        const uint4* vp = reinterpret_cast<const uint4*>(vcodes + (int64_t)tv * RBV + wave * SEGV);
#pragma unroll
        for (int u = 0; u < VB; ++u) in.vq[u] = ld_stream4(vp + u);
        in.nk = kn[(int64_t)tv * nbk];
        in.nv = vn[(int64_t)tv * nbv];
    };
    float* nrm = nrms + wave * 128;  // this wave's K norms [64] then V norms [64] of the tile

    TileIn cur;
    if (t_beg < t_end) fetch(cur, t_beg);
    int par = 0;
    for (int t0 = t_beg; t0 < t_end; t0 += 64, par ^= 1) {
        TileIn nxt;
        fetch(nxt, t0 + 64 < t_end ? t0 + 64 : t0);  // the next tile's loads go out now
        // the tile's norms of this wave's halves, one token per lane (the
        // previous tile's reads of this area are done)
        nrm[lane] = half_bits_to_float(cur.nk) * bs_k;
        nrm[64 + lane] = half_bits_to_float(cur.nv);
        wave_order();
        // ---- partial scores of the wave's quarter: the four 16-token blocks'
        // matrix-core chains interleaved step by step
        float* pw = psc + par * PB + wave * kMcRows * kPStride;
        mf4_t kacc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) kacc[tb] = mf4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint2 e0 = ktl[bits_from<2 * KB>(cur.cw[tb], 4 * ks * KB) * KTS];
                const uint2 e1 = ktl[bits_from<2 * KB>(cur.cw[tb], (4 * ks + 2) * KB) * KTS];
                kacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_mh8(make_uint4(e0.x, e0.y, e1.x, e1.y)), bq[ks],
                                                                 kacc[tb], 0, 0, 0);
            }
        }
        // column n + 8 holds the q_lo part of head n: add the two halves; lanes
        // n < 8 then hold tokens 16 tb + 4 grp + v of head n
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const float4 nk4 = *reinterpret_cast<const float4*>(nrm + 16 * tb + 4 * grp);
            const float nkv[4] = {nk4.x, nk4.y, nk4.z, nk4.w};
            float sv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) sv[v] = (kacc[tb][v] + xor_lane<8>(kacc[tb][v])) * qinv * nkv[v];
            if (n < 8)
                *reinterpret_cast<float4*>(pw + n * kPStride + 16 * tb + 4 * grp) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        }
        __syncthreads();  // every wave's partial scores of the tile are in LDS

        // ---- softmax: lane (n, grp) takes head hq and tokens 32 s2 + 8 grp + e
        const float* pb = psc + par * PB + hq * kPStride;
        float s[2][8];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[s2][e] = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float4* src = reinterpret_cast<const float4*>(pb + w * kMcRows * kPStride + 32 * s2 + 8 * grp);
                const float4 u0 = src[0], u1 = src[1];
                s[s2][0] += u0.x; s[s2][1] += u0.y; s[s2][2] += u0.z; s[s2][3] += u0.w;
                s[s2][4] += u1.x; s[s2][5] += u1.y; s[s2][6] += u1.z; s[s2][7] += u1.w;
            }
        }
        const bool full = t0 + 64 <= t_end;  // uniform: no token past the split's end
        float tmax = -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (!full) s[s2][e] = (t0 + 32 * s2 + 8 * grp + e < t_end) ? s[s2][e] : -INFINITY;
                tmax = fmaxf(tmax, s[s2][e]);
            }
        }
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        const float mn = fmaxf(m, tmax);  // finite: the tile holds a token
        const float f = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first tile (m = -inf)
        float psum = 0.0f;
        uint32_t wa[2][4];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const float4 va = *reinterpret_cast<const float4*>(nrm + 64 + 32 * s2 + 8 * grp);
            const float4 vb = *reinterpret_cast<const float4*>(nrm + 64 + 32 * s2 + 8 * grp + 4);
            const float nv8[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // exp2 of a value <= 0 (-inf past the end gives 0)
                const float p = live_row ? __builtin_amdgcn_exp2f(s[s2][e] - mn) : 0.0f;
                psum += p;
                pe[e] = p * nv8[e];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) wa[s2][j] = pack_halves(pe[2 * j], pe[2 * j + 1]);
        }
        psum += xor_lane<16>(psum);
        psum += xor_lane<32>(psum);
        l = l * f + psum;
        m = mn;
        // rescale the value sums when some head's max rose: rows 4 grp + i hold
        // head 4 grp + i (rows 8..15 are unused), whose factor sits in lane
        // 4 grp + i
        if (__builtin_amdgcn_ballot_w64(f != 1.0f) != 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fi = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * grp + i) << 2, __float_as_int(f)));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) vacc[nb][i] *= fi;
            }
        }

        // ---- stage the value quarters (lane = token); the previous tile's
        // reads of this wave's area are done
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            vs[lane * VSTR + 4 * u] = cur.vq[u].x;
            vs[lane * VSTR + 4 * u + 1] = cur.vq[u].y;
            vs[lane * VSTR + 4 * u + 2] = cur.vq[u].z;
            vs[lane * VSTR + 4 * u + 3] = cur.vq[u].w;
        }
        wave_order();
        // ---- value sums: k step s2 covers tokens 32 s2 + 8 grp + e, column n'
        // stands for dim 8 n' + nb of the quarter
        const int bit0 = PIECE * n, wi = bit0 >> 5, sh = bit0 & 31;
        // V pair table entry of the 2 VB bits at bit fb of a piece: the index
        // lands on the table's row stride with one shift and one and-or
        auto vlook = [&](uint32_t pcv, int fb) __attribute__((always_inline)) {
            const uint32_t sl = fb <= VLOG ? (pcv << (VLOG - fb)) : (pcv >> (fb - VLOG));
            const uint32_t off = (sl & ((VTE - 1u) << VLOG)) | vlane;
            return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(vtab) + off);
        };
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t pc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // dword wi + 1 is at most the row's padding dword; its bits only
                // enter when the piece crosses into it
                const uint32_t* row = vs + (32 * s2 + 8 * grp + e) * VSTR;
                pc[e] = __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh);
            }
            const mh8_t aw = as_mh8(make_uint4(wa[s2][0], wa[s2][1], wa[s2][2], wa[s2][3]));
#pragma unroll
            for (int pp = 0; pp < NB / 2; ++pp) {
                uint32_t ent[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ent[e] = vlook(pc[e], 2 * pp * VB);
                const uint4 blo = make_uint4(__builtin_amdgcn_perm(ent[1], ent[0], 0x05040100u),
                                             __builtin_amdgcn_perm(ent[3], ent[2], 0x05040100u),
                                             __builtin_amdgcn_perm(ent[5], ent[4], 0x05040100u),
                                             __builtin_amdgcn_perm(ent[7], ent[6], 0x05040100u));
                const uint4 bhi = make_uint4(__builtin_amdgcn_perm(ent[1], ent[0], 0x07060302u),
                                             __builtin_amdgcn_perm(ent[3], ent[2], 0x07060302u),
                                             __builtin_amdgcn_perm(ent[5], ent[4], 0x07060302u),
                                             __builtin_amdgcn_perm(ent[7], ent[6], 0x07060302u));
                vacc[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_mh8(blo), vacc[2 * pp], 0, 0, 0);
                vacc[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_mh8(bhi), vacc[2 * pp + 1], 0, 0, 0);
            }
        }
        wave_order();  // every lane has read the staged quarters before the next tile
        cur = nxt;
    }

    // one partial per query row of the block split: (max, sum, acc[D]); the
    // waves agree on (max, sum), wave 0 writes them, each wave its own dims
    if (wave == 0 && grp == 0 && n < G) {
        float* pr = a.part + (((int64_t)b * a.hq + row0 + n) * a.splits + split) * (D + 2);
        pr[0] = m;
        pr[1] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * grp + i;
        if (h < G) {
            float* pr = a.part + (((int64_t)b * a.hq + row0 + h) * a.splits + split) * (D + 2) + 2 + DW * wave + 8 * n;
#pragma unroll
            for (int nb = 0; nb < NB; nb += 2) {
                *reinterpret_cast<float2*>(pr + nb) = make_float2(vacc[nb][i] * bs_v, vacc[nb + 1][i] * bs_v);
            }
        }
    }
}

template <int KB>
void launch_mc_k(const AttnArgs& a, hipStream_t s) {
    const dim3 grid(a.splits, a.hkv * a.chunks, a.batch);
    switch (a.vc.bits) {
        case 1: hipLaunchKernelGGL((wide_mc_kernel<KB, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((wide_mc_kernel<KB, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((wide_mc_kernel<KB, 3>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((wide_mc_kernel<KB, 4>), grid, dim3(256), 0, s, a); break;
    }
}

}  // namespace

hipError_t launch_wide(const AttnArgs& a, hipStream_t s) {
    switch (a.kc.bits) {
        case 1: launch_mc_k<1>(a, s); break;
        case 2: launch_mc_k<2>(a, s); break;
        case 3: launch_mc_k<3>(a, s); break;
        default: launch_mc_k<4>(a, s); break;
    }
    return hipGetLastError();
}

}  // namespace tqi
