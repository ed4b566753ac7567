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
template <int D, int KB, int VB, int G>
struct Cfg {
    static constexpr int RBK = D * KB / 8;          // K code bytes per token
    static constexpr int RBV = D * VB / 8;          // V code bytes per token
    static constexpr int KLU = (KB == 3) ? 6 : 8;   // bits per K table lookup
    static constexpr int KCPL = KLU / KB;           // K codes per lookup
    static constexpr int NKLU = D * KB / KLU;       // lookups per K row
    static constexpr int KFENCE = (8 + KCPL - 1) / KCPL;  // lookups between scheduling fences (8 dims)
    static constexpr int KTAB = (1 << KLU) * KCPL;  // floats in the K table
    static constexpr int VD = D / 64;               // V dims per lane
    static constexpr int VLB = 2 * VB;              // bits per V pair lookup
    static constexpr int VTAB = 1 << VLB;           // float2 entries
    static constexpr int VTDW = 64 * RBV / 4 + 4;   // V tile dwords (+ pad)
    static constexpr int MAIN = 4 * (G * 64 + VTDW);       // per-wave W + V tile (dwords)
    static constexpr int MERGE = 4 * G * (D + 2);           // block merge area (floats)
    static constexpr int UNION = MAIN > MERGE ? MAIN : MERGE;
    static constexpr int SMEM = KTAB + 2 * VTAB + UNION;    // dwords
};

template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(256) void split_kernel(AttnArgs a) {
    using C = Cfg<D, KB, VB, G>;
    __shared__ __attribute__((aligned(16))) float smem[C::SMEM];
    float* ktab = smem;
    float2* vtab = reinterpret_cast<float2*>(smem + C::KTAB);
    float* uni = smem + C::KTAB + 2 * C::VTAB;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.chunks, chunk = blockIdx.y - kvh * a.chunks;
    const int b = blockIdx.z;
    int64_t ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
    const int64_t t_beg = (int64_t)split * a.split_tokens;
    const int64_t t_end = (t_beg + a.split_tokens < ctx) ? t_beg + a.split_tokens : ctx;

    // centroid tables: ktab[u*KCPL + p] = c_K[code p of u], vtab[u] = (c_V[lo], c_V[hi])
    for (int u = tid; u < (1 << C::KLU); u += 256) {
#pragma unroll
        for (int p = 0; p < C::KCPL; ++p) ktab[u * C::KCPL + p] = a.kc.centroid[(u >> (KB * p)) & ((1 << KB) - 1)];
    }
    for (int u = tid; u < C::VTAB; u += 256)
        vtab[u] = make_float2(a.vc.centroid[u & ((1 << VB) - 1)], a.vc.centroid[(u >> VB) & ((1 << VB) - 1)]);
    __syncthreads();

    const int h0 = kvh * a.g + chunk * G;
    const int m = a.kc.qjl_m;
    const float* qrot = a.qrot + ((int64_t)b * a.hq + h0) * D;
    const float* qproj = a.qproj + ((int64_t)b * a.hq + h0) * m;
    const int64_t kvrow = ((int64_t)b * a.hkv + kvh) * a.ctx_cap;
    const uint8_t* kcodes = a.k_codes + kvrow * C::RBK;
    const uint8_t* vcodes = a.v_codes + kvrow * C::RBV;

    float* wbuf = uni + wave * (G * 64 + C::VTDW);
    uint32_t* vtile = reinterpret_cast<uint32_t*>(wbuf + G * 64);

    float m_run[G], l_lane[G], acc[G][C::VD];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_lane[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < C::VD; ++j) acc[h][j] = 0.0f;
    }
    // this lane's V bits inside a row: VD*VB bits at lane*VD*VB
    const int vbit0 = lane * C::VD * VB;
    const int vdw = vbit0 >> 5, vsh = vbit0 & 31;

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    for (int64_t t0 = t_beg + wave_u * 64; t0 < t_end; t0 += 256) {
        const int64_t t = t0 + lane;
        const bool valid = t < t_end;
        uint32_t kw[C::RBK / 4];
        uint32_t vw[C::RBV / 4];
        float kn = 0.0f, vn = 0.0f;
        if (valid) {
            const uint4* kp = reinterpret_cast<const uint4*>(kcodes + t * C::RBK);
#pragma unroll
            for (int j = 0; j < C::RBK / 16; ++j) {
                const uint4 r = kp[j];
                kw[4 * j] = r.x; kw[4 * j + 1] = r.y; kw[4 * j + 2] = r.z; kw[4 * j + 3] = r.w;
            }
            if constexpr (C::RBV % 16 == 0) {
                const uint4* vp = reinterpret_cast<const uint4*>(vcodes + t * C::RBV);
#pragma unroll
                for (int j = 0; j < C::RBV / 16; ++j) {
                    const uint4 r = vp[j];
                    vw[4 * j] = r.x; vw[4 * j + 1] = r.y; vw[4 * j + 2] = r.z; vw[4 * j + 3] = r.w;
                }
            } else {
                const uint2* vp = reinterpret_cast<const uint2*>(vcodes + t * C::RBV);
#pragma unroll
                for (int j = 0; j < C::RBV / 8; ++j) {
                    const uint2 r = vp[j];
                    vw[2 * j] = r.x; vw[2 * j + 1] = r.y;
                }
            }
            kn = half_bits_to_float(a.k_norms[kvrow + t]);
            vn = half_bits_to_float(a.v_norms[kvrow + t]);
        } else {
#pragma unroll
            for (int j = 0; j < C::RBK / 4; ++j) kw[j] = 0u;
#pragma unroll
            for (int j = 0; j < C::RBV / 4; ++j) vw[j] = 0u;
        }
#pragma unroll
        for (int j = 0; j < C::RBV / 4; ++j) vtile[lane * (C::RBV / 4) + j] = vw[j];

        // A loop-variant zero (t0 < 2^62) keeps the uniform query loads inside
        // the tile loop, where they are scalar loads, instead of letting them
        // be hoisted out of it into hundreds of SGPRs.
        const int zero = (int)(t0 >> 62);
        const float* qr = qrot + zero;

        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.0f;
        static_for<C::NKLU>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int bit0 = u * C::KLU, w = bit0 >> 5, sh = bit0 & 31;
            uint32_t field;
            if constexpr (sh + C::KLU <= 32) {
                field = (kw[w] >> sh) & ((1u << C::KLU) - 1u);
            } else {
                field = __builtin_amdgcn_alignbit(kw[w + 1], kw[w], sh) & ((1u << C::KLU) - 1u);
            }
            float cv[C::KCPL];
            if constexpr (C::KCPL == 2) {
                const float2 t2 = reinterpret_cast<const float2*>(ktab)[field];
                cv[0] = t2.x;
                cv[1] = t2.y;
            } else {
#pragma unroll
                for (int p4 = 0; p4 < C::KCPL / 4; ++p4) {
                    const float4 t4 = reinterpret_cast<const float4*>(ktab)[field * (C::KCPL / 4) + p4];
                    cv[4 * p4] = t4.x; cv[4 * p4 + 1] = t4.y; cv[4 * p4 + 2] = t4.z; cv[4 * p4 + 3] = t4.w;
                }
            }
#pragma unroll
            for (int p = 0; p < C::KCPL; ++p) {
#pragma unroll
                for (int h = 0; h < G; ++h) s[h] = fmaf(qr[(u * C::KCPL + p) * G + h], cv[p], s[h]);
            }
            // bound the scalar-register footprint of the query values in flight
            if constexpr ((u + 1) % C::KFENCE == 0) __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] *= kn;

        if (m > 0) {
            // QJL correction: kn * gamma * sum_j qproj_j * (2 bit_j - 1)
            const float gam = valid ? half_bits_to_float(a.k_gamma[kvrow + t]) : 0.0f;
            const uint32_t* qb = reinterpret_cast<const uint32_t*>(a.k_qjl + (kvrow + (valid ? t : 0)) * (m >> 3));
            const float* qp = qproj + zero;
            float corr[G];
#pragma unroll
            for (int h = 0; h < G; ++h) corr[h] = 0.0f;
            for (int wd = 0; wd < (m >> 5); ++wd) {
                const uint32_t bits = valid ? qb[wd] : 0u;
#pragma unroll 8
                for (int i = 0; i < 32; ++i) {
                    const uint32_t neg = ((~bits >> i) & 1u) << 31;
#pragma unroll
                    for (int h = 0; h < G; ++h) corr[h] += as_f(as_u(qp[h * m + wd * 32 + i]) ^ neg);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = fmaf(kn * gam, corr[h], s[h]);
        }

        // online softmax over the tile, per head
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float sv = valid ? s[h] : -INFINITY;
            const float mt = group_max<64>(sv);
            const float mnew = fmaxf(m_run[h], mt);
            const float alpha = exp2f(m_run[h] - mnew);
            const float p = exp2f(sv - mnew);
            l_lane[h] = fmaf(l_lane[h], alpha, p);
#pragma unroll
            for (int j = 0; j < C::VD; ++j) acc[h][j] *= alpha;
            m_run[h] = mnew;
            wbuf[h * 64 + lane] = p * vn;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // V accumulation in the rotated domain, lane <-> VD dims
        const int64_t left = t_end - t0;
        const int nt4 = (int)((left < 64 ? left : 64) + 3) & ~3;
        for (int tt = 0; tt < nt4; tt += 4) {
            float4 w4[G];
#pragma unroll
            for (int h = 0; h < G; ++h) w4[h] = *reinterpret_cast<const float4*>(wbuf + h * 64 + tt);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t* row = vtile + (tt + q) * (C::RBV / 4);
                uint32_t bits;
                if constexpr (VB == 3) {
                    bits = __builtin_amdgcn_alignbit(row[vdw + 1], row[vdw], vsh);
                } else {
                    bits = row[vdw] >> vsh;
                }
#pragma unroll
                for (int pr = 0; pr < C::VD / 2; ++pr) {
                    const float2 cv = vtab[(bits >> (pr * C::VLB)) & ((1u << C::VLB) - 1u)];
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float wv = q == 0 ? w4[h].x : q == 1 ? w4[h].y : q == 2 ? w4[h].z : w4[h].w;
                        acc[h][2 * pr] = fmaf(wv, cv.x, acc[h][2 * pr]);
                        acc[h][2 * pr + 1] = fmaf(wv, cv.y, acc[h][2 * pr + 1]);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // block merge of the four waves
    float l_tot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) l_tot[h] = group_sum<64>(l_lane[h]);
    __syncthreads();
    float* mrg = uni;  // [4][G][D + 2]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float* r = mrg + (wave * G + h) * (D + 2);
        if (lane == 0) {
            r[0] = m_run[h];
            r[1] = l_tot[h];
        }
#pragma unroll
        for (int j = 0; j < C::VD; ++j) r[2 + lane * C::VD + j] = acc[h][j];
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
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(AttnArgs a) {
    __shared__ float x[D];
    const int bh = blockIdx.x;
    const int i = threadIdx.x;
    const float* p = a.part + (int64_t)bh * a.splits * (D + 2);
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, p[(int64_t)s * (D + 2)]);
    float L = 0.0f, acc = 0.0f;
    if (mx != -INFINITY) {
        for (int s = 0; s < a.splits; ++s) {
            const float* ps = p + (int64_t)s * (D + 2);
            const float f = exp2f(ps[0] - mx);
            L = fmaf(ps[1], f, L);
            acc = fmaf(ps[2 + i], f, acc);
        }
    }
    x[i] = L > 0.0f ? acc / L : 0.0f;
    __syncthreads();
    // inverse rotation: D_V H(x) / d
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
        float nv = 0.0f;
        if ((i & h) == 0) nv = x[i] + x[i + h];
        else nv = x[i - h] - x[i];
        __syncthreads();
        x[i] = nv;
        __syncthreads();
    }
    const uint32_t neg = ((a.vc.sign_mask[i >> 5] >> (i & 31)) & 1u) << 31;
    a.out[(int64_t)bh * D + i] = as_f(as_u(x[i] * (1.0f / (float)D)) ^ neg);
}

template <int D, int KB, int VB, int G>
hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
    dim3 grid(a.splits, a.hkv * a.chunks, a.batch);
    hipLaunchKernelGGL((split_kernel<D, KB, VB, G>), grid, dim3(256), 0, s, a);
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
