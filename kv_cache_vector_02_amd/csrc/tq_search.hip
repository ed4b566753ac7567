// Inner-product search with the unbiased TurboQuant estimator, gfx950.
//
//   est(q, t) = n_t ( <q_rot, c[idx_t]>/d + gamma_t sqrt(pi/2)/m <S q_rot/sqrt(d), 2 bit_t - 1> )
//
// written as one float32 product per (query, row) over K = d + m terms:
// A_q = [q_rot/d, sqrt(pi/2)/m S q_rot/sqrt(d)] and B_t = [c[idx_t], gamma_t (2 bit_t - 1)],
// est = n_t <A_q, B_t>.  The vector-search use case is where the QJL estimator's
// unbiasedness pays off (the TurboQuant PyTorch write-up on idea.jsleekr.com,
// "핵심 발견 1 — QJL 레이어를 제거하라": no softmax in vector search).
//
// Launches: qprep (A, stored k-major [d+m][n_q]), scan (grid = DB chunks x
// 32-query tiles; the estimates on the matrix cores, see below, and exact
// per-block top-k lists in LDS), merge (per query, exact top-k over the block
// lists, ordered by estimate descending then id ascending).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace {

using namespace tqd;

constexpr int KMAX = 64;   // largest k (per-block lists hold 32 or 64 entries)

template <int D>
__global__ __launch_bounds__(64) void search_qprep_kernel(SearchArgs a) {
    constexpr int LPV = D / 8;
    constexpr int VPW = 64 / LPV;
    __shared__ float rot[VPW][D];
    const int lane = threadIdx.x;
    const int gl = lane & (LPV - 1), grp = lane / LPV;
    const int qi = blockIdx.x * VPW + grp;
    const bool valid = qi < a.n_q;
    const int m = a.c.qjl_m;
    const uint32_t sbits = (a.c.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
    float v[8];
    if (valid) {
        load8<0>(a.q + (int64_t)qi * D + gl * 8, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e]) ^ (((sbits >> e) & 1u) << 31));
    fwht<LPV>(v, gl);
    if (valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a.qrot[(int64_t)(gl * 8 + e) * a.n_q + qi] = v[e] * (1.0f / (float)D);
    }
    if (m > 0 && a.c.residual != TQ_RES_QJL) {
        // m = D: the SRHT projection H(D2 q_rot) in registers, or Direct
        // Sign's q_rot itself with the constant 1 in place of sqrt(pi/2)/m
        float ps = 1.0f / sqrtf((float)D);
        if (a.c.residual == TQ_RES_SRHT) {
            const uint32_t sbits2 = (a.c.sign_mask2[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = as_f(as_u(v[e]) ^ (((sbits2 >> e) & 1u) << 31));
            fwht<LPV>(v, gl);
            ps *= sqrtf(1.57079632679489662f) / (float)m;
        }
        if (valid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a.qrot[(int64_t)(D + gl * 8 + e) * a.n_q + qi] = v[e] * ps;
        }
    } else if (m > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rot[grp][gl * 8 + e] = v[e];
        __syncthreads();
        const float ps = sqrtf(1.57079632679489662f) / ((float)m * sqrtf((float)D));
        for (int j = gl; j < m; j += LPV) {
            const float* srow = a.S + (int64_t)j * D;
            float acc = 0.0f;
            for (int i = 0; i < D; ++i) acc = fmaf(srow[i], rot[grp][i], acc);
            if (valid) a.qrot[(int64_t)(D + j) * a.n_q + qi] = acc * ps;
        }
    }
}

// --------------------------------------------------------- matrix cores ----
// The same estimator as one matrix-core contraction per (16 rows, 8 queries):
// v_mfma_f32_16x16x32_f16, lane l holding A[l%16][8(l/16) + e], B[8(l/16) + e][l%16]
// and receiving D[4(l/16) + i][l%16].  Rows of A are database rows, columns of
// B are queries.  Float32-exact products come from splitting both operands into
// half hi + lo parts folded into the two MFMA dimensions with room (the decode
// scan's scheme): the eight k slots of a lane hold (c_hi, c_hi, c_lo, c_lo) of
// two dims twice, columns 0..7 hold q_hi and 8..15 q_lo of the wave's 8 queries
// (zero on the c_lo slots), so D[row][n] + D[row][n + 8] is the product
// sum over (c_hi + c_lo)(q_hi + q_lo) without the c_lo q_lo term (below 2^-22).
// Lane group g = l/16 covers dims g*d/4 + [0, d/4): k step ks takes dims
// g*d/4 + 4ks + [0, 4).  The QJL part takes A = 16 (+-1), exact in half,
// with projections j = g*m/4 + 8js + [0, 8) per k step, accumulated apart
// from the centroid part; the row's gamma multiplies that float32 sum.  Centroids are scaled by
// 16 and each wave's queries by one power of two into [2^14, 2^15) so every lo
// part is a normal half; the scale comes off the float32 result.
//
// A block of 4 waves takes 32 queries (8 per wave, their operands kept in
// registers) and a range of database rows in tiles of 64 staged through LDS
// (rows padded so that the 16 rows a step reads sit on distinct banks); each
// wave scores the tile's rows 16 at a time for its queries.  A lane keeps its
// query's k-th best score in a register, so a group of 16 rows costs one
// compare per score and a wave vote, and only rows above that score go
// through the query's exact top-k list in LDS.
typedef _Float16 sh8_t __attribute__((ext_vector_type(8)));
typedef float sf4_t __attribute__((ext_vector_type(4)));

constexpr int MQ = 32;  // queries per block
constexpr int MT = 64;  // database rows per tile

__device__ __forceinline__ sh8_t as_sh8(uint4 u) { return __builtin_bit_cast(sh8_t, u); }

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// bits [bit0, bit0 + NB) of a little-endian dword array (bit0 compile-time after unrolling)
template <int NB>
__device__ __forceinline__ uint32_t bits_at(const uint32_t* w, int bit0) {
    const int wi = bit0 >> 5, sh = bit0 & 31;
    if (sh + NB <= 32) return (w[wi] >> sh) & ((1u << NB) - 1u);
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << NB) - 1u);
}

__device__ __forceinline__ float wmax64(float v) {
    v = fmaxf(v, xor_lane<1>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<16>(v));
    return fmaxf(v, xor_lane<32>(v));
}

template <int D, int BITS, int KM>
// Three waves per SIMD (168 registers); at d = 256 the variants other than
// 3 bits spill there and take two.  The 3-bit variants with lists of 32 and 64
// keep 12 and 20 bytes in scratch at three waves, which runs faster than two
// waves without them (5.0 against 5.7 ms for 1024 queries over 2^20 rows).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 256 && BITS != 3 ? 2 : 3))) void search_mfma_kernel(
    SearchArgs a) {
    constexpr int RB = D * BITS / 8;   // code bytes per row (a multiple of 16)
    constexpr int RW = RB / 4;         // ... dwords
    // LDS row stride of the staged codes: RW + 2 = 2 x odd, so the 16 rows a
    // sub-tile reads at once start on distinct even banks
    constexpr int RWP = RW + 2;
    constexpr int RV = RB / 16;        // 16-byte pieces per row
    constexpr int NV = MT * RV;        // ... per tile
    constexpr int BWP = 9;             // LDS row stride of the sign bits (<= 8 dwords used), dwords
    constexpr int KP = KM + 1;         // list stride: the 8 lists of a wave on distinct banks
    constexpr int DG = D / 4;          // dims per lane group
    constexpr int KS = DG / 4;         // centroid k steps
    constexpr int GW = DG * BITS / 32; // code dwords per lane group and row
    constexpr int TE = 1 << (2 * BITS);
    // bank-sliced tables: entry e occupies a row of TS copies, lane l reads copy
    // l % TS, so the 32 lanes of a pass hit distinct banks whatever their
    // entries (at 4 bits 8 copies keep the table at 16 KB)
    constexpr int TS = BITS <= 3 ? 32 : 8;
    const int m = a.c.qjl_m;
    // QJL k steps (<= 8); also the sign bytes of a lane group's m/4 projections
    // and the sign dwords of a row
    const int JS = m >> 5;
    const int k = a.k;
    __shared__ __attribute__((aligned(16))) uint2 tab[TE * TS];  // two codes: hi a, hi b | lo a, lo b (of 16 c)
    __shared__ __attribute__((aligned(16))) uint2 sgn[16 * 32];  // nibble -> 4 halves of +-16, 32 copies
    __shared__ __attribute__((aligned(16))) uint32_t rcode[MT * RWP];
    __shared__ __attribute__((aligned(16))) uint32_t rbits[MT * BWP];
    __shared__ __attribute__((aligned(16))) float rn[MT];
    __shared__ __attribute__((aligned(16))) float rg[MT];
    __shared__ float es[MQ][17];       // candidate scores of one sub-tile (16 rows)
    __shared__ float lst_s[MQ * KP];
    __shared__ int32_t lst_i[MQ * KP];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;
    const int q0 = blockIdx.y * MQ;
    const int64_t r_beg = (int64_t)blockIdx.x * a.block_rows;
    const int64_t r_end = (r_beg + a.block_rows < a.n_db) ? r_beg + a.block_rows : a.n_db;

    for (int i = tid; i < TE * TS; i += 256) {
        const int e = i / TS;
        const float fa = 16.0f * a.c.centroid[e & ((1 << BITS) - 1)];
        const float fb = 16.0f * a.c.centroid[e >> BITS];
        const float ha = (float)(_Float16)fa, hb = (float)(_Float16)fb;
        tab[i] = make_uint2(pack_h2(ha, hb), pack_h2(fa - ha, fb - hb));
    }
    for (int i = tid; i < 16 * 32; i += 256) {
        const int x = i >> 5;
        auto sg = [&](int b) { return ((x >> b) & 1) ? 16.0f : -16.0f; };
        sgn[i] = make_uint2(pack_h2(sg(0), sg(1)), pack_h2(sg(2), sg(3)));
    }
    const uint2* tabl = tab + lane % TS;  // this lane's table copies
    const uint2* sgnl = sgn + (lane & 31);
    for (int e = tid; e < MQ * KP; e += 256) {
        lst_s[e] = -INFINITY;
        lst_i[e] = -1;
    }

    // this wave's query operands: column n <-> query q0 + 8 wave + (n & 7), hi (n < 8) or lo
    const int qi = q0 + 8 * wave + (n & 7);
    const bool qok = qi < a.n_q;
    const bool lo_col = n >= 8;
    sh8_t bq[KS], bj[8];
    float qinv;
    {
        float amax = 0.0f;
        for (int t = 0; t < DG; ++t) amax = fmaxf(amax, qok ? fabsf(a.qrot[(int64_t)(grp * DG + t) * a.n_q + qi]) : 0.0f);
        for (int t = 0; t < (m >> 2); ++t)
            amax = fmaxf(amax, qok ? fabsf(a.qrot[(int64_t)(D + grp * (m >> 2) + t) * a.n_q + qi]) : 0.0f);
        amax = wmax64(amax);
        float sc = 1.0f;
        if (amax > 0.0f && isfinite(amax)) {
            int ex;
            frexpf(amax, &ex);
            sc = ldexpf(1.0f, 15 - ex);
        }
        qinv = 1.0f / (16.0f * sc);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = qok ? a.qrot[(int64_t)(grp * DG + 4 * ks + i) * a.n_q + qi] * sc : 0.0f;
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
#pragma unroll
        for (int js = 0; js < 8; ++js) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = 0.0f;
                if (js < JS && qok) v = a.qrot[(int64_t)(D + grp * (m >> 2) + 8 * js + e) * a.n_q + qi] * sc;
                const float h = (float)(_Float16)v;
                bj[js][e] = (_Float16)(lo_col ? v - h : h);
            }
        }
    }

    // k-th best score so far of this lane's query (n & 7); only larger scores
    // can enter its list
    float thr = -INFINITY;
    const int ql = 8 * wave + (n & 7);
    for (int64_t t0 = r_beg; t0 < r_end; t0 += MT) {
        const int nt = (int)((r_end - t0) < MT ? (r_end - t0) : MT);
        __syncthreads();  // the previous tile's rows are no longer read
        {
            // the tile's code rows are contiguous in memory: 16-byte pieces
            // into rows of RWP dwords
            const uint4* src = reinterpret_cast<const uint4*>(a.codes + t0 * RB);
            const int nv = nt * RV;
#pragma unroll
            for (int i = 0; i < (NV + 255) / 256; ++i) {
                const int e = tid + 256 * i;
                if (NV % 256 == 0 || e < NV) {
                    const uint4 v = e < nv ? src[e] : make_uint4(0u, 0u, 0u, 0u);
                    const int row = e / RV, c = e - row * RV;
                    uint2* dst = reinterpret_cast<uint2*>(rcode + row * RWP + 4 * c);
                    dst[0] = make_uint2(v.x, v.y);
                    dst[1] = make_uint2(v.z, v.w);
                }
            }
        }
        if (JS > 0) {
            // four threads per row, sign dwords w and w + 4
            const int row = tid >> 2;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(a.qjl + (t0 + row) * (int64_t)(m >> 3));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int w = (tid & 3) + 4 * h;
                if (w < JS) rbits[row * BWP + w] = row < nt ? src[w] : 0u;
            }
        }
        if (tid < MT) {
            rn[tid] = tid < nt ? half_bits_to_float(a.norms[t0 + tid]) : 0.0f;
        } else if (tid < 2 * MT) {
            const int r = tid - MT;
            rg[r] = (r < nt && m > 0) ? half_bits_to_float(a.gamma[t0 + r]) : 0.0f;
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < 4 && 16 * j < nt; ++j) {
            const int r = 16 * j + n;  // this lane's row of the A side
            uint32_t cw[GW];
#pragma unroll
            for (int w = 0; w < GW; ++w) cw[w] = rcode[r * RWP + grp * GW + w];
            // two centroid accumulators (even and odd k steps) and the QJL one:
            // independent matrix-core chains.  The QJL part takes A = 16 (+-1):
            // the row's gamma multiplies its float32 result instead of the
            // operands.  Step js takes the projections of sign byte
            // grp * JS + js of the row.
            sf4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, accq = acc0;
            auto centroid_step = [&](int ks, sf4_t& acc) {
                const uint2 e0 = tabl[bits_at<2 * BITS>(cw, 4 * ks * BITS) * TS];
                const uint2 e1 = tabl[bits_at<2 * BITS>(cw, (4 * ks + 2) * BITS) * TS];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_sh8(make_uint4(e0.x, e0.y, e1.x, e1.y)), bq[ks], acc, 0, 0, 0);
            };
            auto qjl_step = [&](int js, uint32_t lo4, uint32_t hi4) {
                const uint2 lo = sgnl[lo4 * 32], hi = sgnl[hi4 * 32];
                accq = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_sh8(make_uint4(lo.x, lo.y, hi.x, hi.y)), bj[js], accq, 0, 0, 0);
            };
            if (JS == 8) {
                // all eight steps, with no branch: the lane's 8 sign bytes in two
                // dwords, steps interleaved with the centroid ones
                const uint32_t sw[2] = {rbits[r * BWP + 2 * grp], rbits[r * BWP + 2 * grp + 1]};
                auto full_qjl = [&](int js) {
                    const uint32_t w = sw[js >> 2];
                    const int sh = 8 * (js & 3);
                    qjl_step(js, (w >> sh) & 15u, (w >> (sh + 4)) & 15u);
                };
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    centroid_step(ks, (ks & 1) ? acc1 : acc0);
                    if ((ks & 1) && (ks >> 1) < 8) full_qjl(ks >> 1);
                }
#pragma unroll
                for (int js = KS / 2; js < 8; ++js) full_qjl(js);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) centroid_step(ks, (ks & 1) ? acc1 : acc0);
                const uint8_t* sb = reinterpret_cast<const uint8_t*>(rbits + r * BWP) + grp * JS;
#pragma unroll
                for (int js = 0; js < 8; ++js) {
                    if (js < JS) {
                        const uint32_t byte = sb[js];
                        qjl_step(js, byte & 15u, byte >> 4);
                    }
                }
            }
            sf4_t acc = acc0 + acc1;
            // column n + 8 holds the q_lo part of query n: add the two halves
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc[v] += xor_lane<8>(acc[v]);
                accq[v] += xor_lane<8>(accq[v]);
            }
            // lanes n < 8: estimates of rows 16 j + 4 grp + v for query n
            const float4 n4 = *reinterpret_cast<const float4*>(rn + 16 * j + 4 * grp);
            const float4 g4 = *reinterpret_cast<const float4*>(rg + 16 * j + 4 * grp);
            const float nv4[4] = {n4.x, n4.y, n4.z, n4.w}, gv4[4] = {g4.x, g4.y, g4.z, g4.w};
            float s[4];
            uint32_t f = 0;  // bit v: row 4 grp + v beats the list's k-th score
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * j + 4 * grp + v;
                s[v] = (n < 8 && row < nt) ? nv4[v] * (fmaf(gv4[v], accq[v], acc[v]) * qinv) : -INFINITY;
                f |= (s[v] > thr ? 1u : 0u) << v;
            }
            if (__builtin_amdgcn_ballot_w64(f != 0) == 0) continue;  // no candidate in the wave: the common case
            // exact top-k insertion of the candidates, in row order (score
            // desc, id asc; ids grow along the scan, so an equal score never
            // displaces an entry)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if ((f >> v) & 1u) es[ql][4 * grp + v] = s[v];
            // candidate rows of query n (bit 4 grp + v) gathered from lanes n + 16 grp
            uint32_t mk = f | (xor_lane_u<16>(f) << 4);
            mk |= xor_lane_u<32>(mk) << 8;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float kth = -INFINITY;
            if (lane < 8) {
                float* ls = lst_s + ql * KP;
                int32_t* li = lst_i + ql * KP;
                while (mk != 0) {
                    const int i = __builtin_ctz(mk);
                    mk &= mk - 1u;
                    const float sc = es[ql][i];
                    if (sc > ls[k - 1]) {
                        int pos = k - 1;
                        while (pos > 0 && ls[pos - 1] < sc) {
                            ls[pos] = ls[pos - 1];
                            li[pos] = li[pos - 1];
                            --pos;
                        }
                        ls[pos] = sc;
                        li[pos] = (int32_t)(t0 + 16 * j + i);
                    }
                }
                kth = ls[k - 1];
            }
            // every lane of query n takes its new k-th score from lane n & 7
            thr = __int_as_float(__builtin_amdgcn_ds_bpermute((n & 7) << 2, __float_as_int(kth)));
        }
    }
    __syncthreads();
    for (int e = tid; e < MQ * k; e += 256) {
        const int q = e / k, jj = e % k;
        if (q0 + q < a.n_q) {
            const int64_t o = ((int64_t)(q0 + q) * a.n_blocks + blockIdx.x) * k + jj;
            a.cand_s[o] = lst_s[q * KP + jj];
            a.cand_i[o] = lst_i[q * KP + jj];
        }
    }
}

// Exact top-k of one query over all block candidates: k rounds of a block-wide
// arg-max under the order (score desc, id asc), ids -1 (empty slots) last.
__global__ __launch_bounds__(256) void search_merge_kernel(SearchArgs a) {
    const int q = blockIdx.x;
    const int nc = a.n_blocks * a.k;
    const float* cs = a.cand_s + (int64_t)q * nc;
    const int32_t* ci = a.cand_i + (int64_t)q * nc;
    __shared__ float bs[256];
    __shared__ int32_t bi[256], bp[256];
    __shared__ int taken[KMAX];
    const int tid = threadIdx.x;
    for (int r = 0; r < a.k; ++r) {
        float best = -INFINITY;
        int32_t bid = -1, bpos = -1;
        for (int c = tid; c < nc; c += 256) {
            bool used = false;
            for (int u = 0; u < r; ++u) used |= taken[u] == c;
            if (used) continue;
            const float s = cs[c];
            const int32_t id = ci[c];
            if (id < 0) continue;
            const bool better = bpos < 0 || s > best || (s == best && id < bid);
            if (better) {
                best = s;
                bid = id;
                bpos = c;
            }
        }
        bs[tid] = best;
        bi[tid] = bid;
        bp[tid] = bpos;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) {
                const int o = tid + w;
                const bool ob = bp[o] >= 0 && (bp[tid] < 0 || bs[o] > bs[tid] || (bs[o] == bs[tid] && bi[o] < bi[tid]));
                if (ob) {
                    bs[tid] = bs[o];
                    bi[tid] = bi[o];
                    bp[tid] = bp[o];
                }
            }
            __syncthreads();
        }
        if (tid == 0) {
            taken[r] = bp[0];
            a.out_scores[(int64_t)q * a.k + r] = bp[0] >= 0 ? bs[0] : -INFINITY;
            a.out_ids[(int64_t)q * a.k + r] = bp[0] >= 0 ? (int64_t)bi[0] : -1;
        }
        __syncthreads();
    }
}

template <int D, int KM>
hipError_t launch_scan_k(const SearchArgs& a, hipStream_t s) {
    const dim3 grid(a.n_blocks, (a.n_q + MQ - 1) / MQ);
    switch (a.c.bits) {
        case 1: hipLaunchKernelGGL((search_mfma_kernel<D, 1, KM>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((search_mfma_kernel<D, 2, KM>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((search_mfma_kernel<D, 3, KM>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((search_mfma_kernel<D, 4, KM>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

// per-block lists of 32 entries for k <= 32 (less LDS per block), else 64
template <int D>
hipError_t launch_scan_b(const SearchArgs& a, hipStream_t s) {
    return a.k <= 32 ? launch_scan_k<D, 32>(a, s) : launch_scan_k<D, KMAX>(a, s);
}

}  // namespace

// Resident scan blocks per compute unit for this variant (cached; 0 without a device).
static int search_blocks(int d, int bits, int k) {
    static std::atomic<int> cache[2][4][2];
    std::atomic<int>& c = cache[d == 256 ? 1 : 0][bits - 1][k <= 32 ? 0 : 1];
    int nb = c.load(std::memory_order_relaxed);
    if (nb > 0) return nb;
    const void* f = nullptr;
    auto pick = [&](auto dk) {
        constexpr int D = decltype(dk)::value;
        if (k <= 32) {
            switch (bits) {
                case 1: f = (const void*)search_mfma_kernel<D, 1, 32>; break;
                case 2: f = (const void*)search_mfma_kernel<D, 2, 32>; break;
                case 3: f = (const void*)search_mfma_kernel<D, 3, 32>; break;
                default: f = (const void*)search_mfma_kernel<D, 4, 32>; break;
            }
        } else {
            switch (bits) {
                case 1: f = (const void*)search_mfma_kernel<D, 1, KMAX>; break;
                case 2: f = (const void*)search_mfma_kernel<D, 2, KMAX>; break;
                case 3: f = (const void*)search_mfma_kernel<D, 3, KMAX>; break;
                default: f = (const void*)search_mfma_kernel<D, 4, KMAX>; break;
            }
        }
    };
    if (d == 256) pick(std::integral_constant<int, 256>{});
    else pick(std::integral_constant<int, 128>{});
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, 256, 0) != hipSuccess || nb <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    c.store(nb, std::memory_order_relaxed);
    return nb;
}

// Database rows per block: a multiple of 64, as many as give one round of
// blocks over the device's resident block slots (compute units x blocks per
// unit for this variant) across the ceil(n_q / 32) query tiles.  A block's
// fixed costs (its query operands, list setup and write-out, and the early
// insertions while its lists fill) shrink per row as the block grows, so the
// fewest blocks that still occupy every slot are the fastest (measured on the
// 2^20 x 256 database with 1024 queries: 4096 rows per block 7.4 ms, two
// rounds 5.2 ms, one round 4.9 ms).  At most 4096 / k blocks, so the merge
// sees at most 4096 candidates per query.  The plan depends on the current
// device.
void search_plan(int n_q, int64_t n_db, int k, int d, int bits, int* n_blocks, int64_t* block_rows) {
    const int64_t qt = ((int64_t)(n_q > 0 ? n_q : 1) + MQ - 1) / MQ;
    const int per_cu = search_blocks(d, bits, k);
    const int64_t slots = (int64_t)device_cus() * (per_cu > 0 ? per_cu : 1);
    const int64_t max_nb = 4096 / (k > 0 ? k : 1);
    int64_t nb = (slots + qt - 1) / qt;
    nb = nb < 1 ? 1 : (nb > max_nb ? max_nb : nb);
    int64_t rows = ((n_db + nb - 1) / nb + 63) & ~(int64_t)63;
    if (rows < 64) rows = 64;
    nb = (n_db + rows - 1) / rows;
    if (nb < 1) nb = 1;
    // A positive TQ_SEARCH_ROWS in the environment replaces the rows per block
    // (rounded up to a multiple of 64, within the candidate bound above); read
    // per call, so the workspace query and the call that follows agree.
    if (const char* env = getenv("TQ_SEARCH_ROWS")) {
        const long want = strtol(env, nullptr, 10);
        if (want > 0) {
            const int64_t r = ((int64_t)want + 63) & ~(int64_t)63;
            const int64_t b2 = (n_db + r - 1) / r;
            if (b2 <= max_nb) {
                rows = r;
                nb = b2 < 1 ? 1 : b2;
            }
        }
    }
    *n_blocks = (int)nb;
    *block_rows = rows;
}

size_t search_workspace(int n_q, int d, int m, int k, int n_blocks) {
    const size_t qa = ((size_t)n_q * (d + m) + 63) & ~(size_t)63;
    const size_t cand = (size_t)n_q * n_blocks * k;
    const size_t candr = (cand + 63) & ~(size_t)63;
    return (qa + 2 * candr) * sizeof(float);
}

hipError_t launch_search(const SearchArgs& a, hipStream_t s) {
    constexpr int VPW128 = 64 / 16, VPW256 = 64 / 32;
    if (a.c.d == 128)
        hipLaunchKernelGGL((search_qprep_kernel<128>), dim3((a.n_q + VPW128 - 1) / VPW128), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((search_qprep_kernel<256>), dim3((a.n_q + VPW256 - 1) / VPW256), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = a.c.d == 128 ? launch_scan_b<128>(a, s) : launch_scan_b<256>(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(search_merge_kernel, dim3(a.n_q), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace tqi
