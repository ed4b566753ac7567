// Decode attention over caches with two norm blocks at head dimension 256,
// which the matrix-core scan does not serve (one norm per half of the
// rotated vector, "TurboQuant KV 캐시 압축 for llama.cpp", v1.5.2 "핵심 변경" item
// 5).  The kernel is generic in D (256 and 512).  The scan's matrix-core
// operations sum the dims of all four quarters of a token in one instruction,
// so a norm per half cannot enter there; this kernel runs on the vector ALUs.
//
// Grid (splits, kv head x head chunk, batch), 4 waves per block taking the
// split's 64-token tiles in turn; the waves merge their states through LDS and
// the block writes one partial (max, sum, acc[d]) per row in the layout the
// combine kernel merges.
// Per 64-token tile of a wave:
//   * scores, lane = token: the token's K codes (32 codes per load) against
//     the block's rotated queries in LDS (broadcast reads),
//     one float32 sum per head and norm block, scaled by the block's norm;
//   * online softmax per head across the wave in log2 units;
//   * value sums, lane = 8 (d = 512) or 4 (d = 256) dims: the tile's V rows
//     (loaded by their token's lane at the start of the tile, in flight during
//     the scores) staged in the wave's LDS tile, then the tokens one at a
//     time, weights and V norms broadcast from the lane that scored the
//     token; sums stay in the rotated domain (one inverse transform per output
//     row in the combine).
#include <hip/hip_runtime.h>
#include <math.h>

#include <utility>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace {

using namespace tqd;

constexpr float kLog2eW = 1.4426950408889634f;
constexpr int kWideRows = 8;  // query rows per block at most

__device__ __forceinline__ float wave_max64(float v) {
    v = fmaxf(v, xor_lane<1>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<16>(v));
    return fmaxf(v, xor_lane<32>(v));
}

__device__ __forceinline__ float bcast(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BITS>
__device__ __forceinline__ uint32_t field(const uint32_t* w, int bit0) {
    const int wi = bit0 >> 5, sh = bit0 & 31;
    if (sh + BITS <= 32) return (w[wi] >> sh) & ((1u << BITS) - 1u);
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << BITS) - 1u);
}

// GR (4 or 8) query rows are computed, rows G..GR-1 with zero queries: no
// per-row branch inside the token loops, so their loads and FMAs pipeline.
template <int D, int KB, int VB, int GR>
__global__ __launch_bounds__(256) void wide_kernel(AttnArgs a) {
    constexpr int LPV = D / 8;          // lanes of one query row in the rotation
    constexpr int RPW = 64 / LPV;       // query rows per wave pass of the rotation
    constexpr int RBK = D * KB / 8;     // K code bytes per token
    constexpr int RBV = D * VB / 8;     // V code bytes per token
    constexpr int DPL = D / 64;         // value dims per lane
    constexpr int PBITS = DPL * VB;     // a lane's value bits of one token (<= 32)
    static_assert(RBK % 4 == 0 && RBV % 8 == 0 && PBITS <= 32, "row layout");
    constexpr int VW = RBV / 4;          // dwords of a V row
    constexpr int VSTR = VW + 1;         // padded stride of the staged rows (odd: no bank conflicts)
    // LDS: rotated queries, then the 4 waves' V tiles; after the token loop the
    // same space holds the states of two waves for the block merge
    constexpr int LOOP_DW = kWideRows * D + 4 * 64 * VSTR;
    constexpr int MERGE_DW = 2 * kWideRows * (D + 2);
    static_assert(MERGE_DW <= LOOP_DW, "merge area exceeds the loop space");
    __shared__ __attribute__((aligned(16))) uint32_t smem[LOOP_DW];
    __shared__ float cent[32];
    float* qr = reinterpret_cast<float*>(smem);
    uint32_t* vtile = smem + kWideRows * D;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

    if (tid < 16) cent[tid] = a.kc.centroid[tid];
    else if (tid < 32) cent[tid] = a.vc.centroid[tid - 16];
    // rotated queries qr[r][i] = (scale log2(e) / d) H(D_K q_r)
    for (int r0 = wave * RPW; r0 < GR; r0 += 4 * RPW) {
        const int r = r0 + lane / LPV, gl = lane & (LPV - 1);
        float x[8];
        if (r < G) {
            const int64_t e0 = ((int64_t)b * a.hq + row0 + r) * D + 8 * gl;
            if (a.q_dtype == TQ_F32) load8<0>(static_cast<const float*>(a.q) + e0, x);
            else if (a.q_dtype == TQ_F16) load8<1>(static_cast<const uint16_t*>(a.q) + e0, x);
            else load8<2>(static_cast<const uint16_t*>(a.q) + e0, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
        const uint32_t sb = (a.kc.sign_mask[gl >> 2] >> ((gl & 3) * 8)) & 0xFFu;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = as_f(as_u(x[e]) ^ (((sb >> e) & 1u) << 31));
        fwht<LPV>(x, gl);
        const float qs = a.scale * kLog2eW / (float)D;
        if (r < GR) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qr[r * D + 8 * gl + e] = x[e] * qs;
        }
    }
    __syncthreads();

    const int nbk = a.kc.norm_blocks, nbv = a.vc.norm_blocks;
    const float bs_k = nbk == 2 ? 1.41421356237309505f : 1.0f;  // sqrt(B)
    const float bs_v = nbv == 2 ? 1.41421356237309505f : 1.0f;
    const uint16_t* kn = a.k_norms + kvrow * nbk;
    const uint16_t* vn = a.v_norms + kvrow * nbv;
    const uint8_t* kcodes = a.k_codes + kvrow * RBK;
    const uint8_t* vcodes = a.v_codes + kvrow * RBV;
    const int vblk = (nbv == 2 && lane >= 32) ? 1 : 0;  // norm block of this lane's value dims
    const int pbit = PBITS * lane;                      // this lane's value bits in a row

    float m[GR], l[GR], acc[GR][DPL];
#pragma unroll
    for (int h = 0; h < GR; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.0f;
    }

    uint32_t* vt = vtile + wave * 64 * VSTR;
    for (int t0 = t_beg + wave * 64; t0 < t_end; t0 += 256) {
        const int t = t0 + lane;
        const bool valid = t < t_end;
        const int tl = valid ? t : t_end - 1;
        // this token's V row: loads out now, into the wave's LDS tile after
        // the scores (the value loop then reads every token's row from LDS)
        uint32_t vrow[VW];
        {
            const uint2* vp = reinterpret_cast<const uint2*>(vcodes + (int64_t)tl * RBV);
#pragma unroll
            for (int u = 0; u < VW / 2; ++u) {
                const uint2 v = ld_stream2(vp + u);
                vrow[2 * u] = v.x;
                vrow[2 * u + 1] = v.y;
            }
        }
        // ---- scores (lane = token), one sum per head and norm block.  The
        // token's K row is read in groups of 32 codes (KB dwords); inside a
        // group the code fields sit at compile-time bit offsets.
        float s0[GR], s1[GR];
#pragma unroll
        for (int h = 0; h < GR; ++h) s0[h] = s1[h] = 0.0f;
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(kcodes + (int64_t)tl * RBK);
        for (int grp = 0; grp < D / 32; ++grp) {
            uint32_t w[KB];
            if constexpr (KB == 4) {
                const uint4 v = ld_stream4(kp + 4 * grp);
                w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            } else if constexpr (KB == 2) {
                const uint2 v = ld_stream2(kp + 2 * grp);
                w[0] = v.x; w[1] = v.y;
            } else {
#pragma unroll
                for (int u = 0; u < KB; ++u) w[u] = ld_stream1(kp + KB * grp + u);
            }
            float part[GR];
#pragma unroll
            for (int h = 0; h < GR; ++h) part[h] = 0.0f;
            const float* qg = qr + 32 * grp;
            static_for<8>([&](auto fc) __attribute__((always_inline)) {
                constexpr int f = decltype(fc)::value;  // four codes 4f .. 4f + 3
                float c[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) c[k] = cent[field<KB>(w, KB * (4 * f + k))];
#pragma unroll
                for (int h = 0; h < GR; ++h) {
                    const float4 q4 = *reinterpret_cast<const float4*>(qg + h * D + 4 * f);
                    float ph = part[h];
                    ph = fmaf(q4.x, c[0], ph);
                    ph = fmaf(q4.y, c[1], ph);
                    ph = fmaf(q4.z, c[2], ph);
                    ph = fmaf(q4.w, c[3], ph);
                    part[h] = ph;
                }
            });
            const bool second = grp >= D / 64;  // the group's norm block (uniform)
#pragma unroll
            for (int h = 0; h < GR; ++h) {
                s0[h] += second ? 0.0f : part[h];
                s1[h] += second ? part[h] : 0.0f;
            }
        }
        // block norms (half values) of this lane's token
        float n0, n1;
        if (nbk == 2) {
            n0 = half_bits_to_float(kn[2 * (int64_t)tl]) * bs_k;
            n1 = half_bits_to_float(kn[2 * (int64_t)tl + 1]) * bs_k;
        } else {
            n0 = n1 = half_bits_to_float(kn[tl]);
        }
        float vs0, vs1;
        if (nbv == 2) {
            vs0 = half_bits_to_float(vn[2 * (int64_t)tl]) * bs_v;
            vs1 = half_bits_to_float(vn[2 * (int64_t)tl + 1]) * bs_v;
        } else {
            vs0 = vs1 = half_bits_to_float(vn[tl]);
        }
        // ---- online softmax per head across the wave
        float p[GR];
#pragma unroll
        for (int h = 0; h < GR; ++h) {
            p[h] = 0.0f;
            const float sc = valid ? fmaf(s0[h], n0, s1[h] * n1) : -INFINITY;
            const float mn = fmaxf(m[h], wave_max64(sc));
            if (mn != -INFINITY) {
                const float f = exp2f(m[h] - mn);  // 0 when m was -inf
                l[h] *= f;
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] *= f;
                p[h] = valid ? exp2f(sc - mn) : 0.0f;
                l[h] += p[h];
                m[h] = mn;
            }
        }
        // ---- value sums (lane = dims), the tile's tokens in order
        // (the wave's previous tile is consumed: its rows can be replaced)
#pragma unroll
        for (int w = 0; w < VW; ++w) vt[lane * VSTR + w] = vrow[w];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int nt = t_end - t0 < 64 ? t_end - t0 : 64;
        const int wi = pbit >> 5, sh = pbit & 31;
        for (int j = 0; j < nt; ++j) {
            // the lane's PBITS bits of token j's row (one staged row read by
            // the whole wave: consecutive dwords, no bank conflicts)
            const uint32_t lo = vt[j * VSTR + wi];
            const uint32_t hi = (sh + PBITS > 32) ? vt[j * VSTR + wi + 1] : 0u;
            const uint32_t bits = sh ? __builtin_amdgcn_alignbit(hi, lo, sh) : lo;
            // token j's norm of this lane's block: both broadcast, then chosen
            const float v0j = bcast(vs0, j), v1j = bcast(vs1, j);
            const float vsj = vblk ? v1j : v0j;
            float vv[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) vv[e] = cent[16 + ((bits >> (VB * e)) & ((1u << VB) - 1u))] * vsj;
#pragma unroll
            for (int h = 0; h < GR; ++h) {
                const float pj = bcast(p[h], j);
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(pj, vv[e], acc[h][e]);
            }
        }
        // every lane has read the tile before any lane overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- block merge of the 4 waves' (max, sum, acc) in two pairwise rounds
    // through LDS (waves 2, 3 into 0, 1; then 1 into 0), then one partial per
    // row of the block split: (max, sum, acc[D]) in the combine's layout
#pragma unroll
    for (int h = 0; h < GR; ++h) {
        float lh = l[h];
        lh += xor_lane<1>(lh);
        lh += xor_lane<2>(lh);
        lh += xor_lane<4>(lh);
        lh += xor_lane<8>(lh);
        lh += xor_lane<16>(lh);
        l[h] = lh + xor_lane<32>(lh);
    }
    float* mrg = reinterpret_cast<float*>(smem);  // [2][kWideRows][D + 2]
    auto put = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < GR; ++h) {
            float* st = mrg + (slot * kWideRows + h) * (D + 2);
            if (lane == 0) {
                st[0] = m[h];
                st[1] = l[h];
            }
#pragma unroll
            for (int e = 0; e < DPL; ++e) st[2 + DPL * lane + e] = acc[h][e];
        }
    };
    auto take = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < GR; ++h) {
            const float* st = mrg + (slot * kWideRows + h) * (D + 2);
            const float mo = st[0], lo = st[1];
            const float mn = fmaxf(m[h], mo);
            if (mn != -INFINITY) {
                const float f = exp2f(m[h] - mn), fo = exp2f(mo - mn);
                l[h] = l[h] * f + lo * fo;
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] = acc[h][e] * f + st[2 + DPL * lane + e] * fo;
                m[h] = mn;
            }
        }
    };
    __syncthreads();  // every wave is done with the queries and its tile
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) take(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);
#pragma unroll
    for (int h = 0; h < GR; ++h) {
        if (h >= G) break;
        float* pr = a.part + (((int64_t)b * a.hq + row0 + h) * a.splits + split) * (D + 2);
        if (lane == 0) {
            pr[0] = m[h];
            pr[1] = l[h];
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) pr[2 + DPL * lane + e] = acc[h][e];
    }
}

template <int D, int KB, int GR>
void launch_wide_g(const AttnArgs& a, hipStream_t s) {
    const dim3 grid(a.splits, a.hkv * a.chunks, a.batch);
    switch (a.vc.bits) {
        case 1: hipLaunchKernelGGL((wide_kernel<D, KB, 1, GR>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((wide_kernel<D, KB, 2, GR>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((wide_kernel<D, KB, 3, GR>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((wide_kernel<D, KB, 4, GR>), grid, dim3(256), 0, s, a); break;
    }
}

// rows computed per block: 4 for chunks of up to 4 query heads, else 8
template <int D, int KB>
hipError_t launch_wide_k(const AttnArgs& a, hipStream_t s) {
    if (a.heads_per_chunk <= 4) launch_wide_g<D, KB, 4>(a, s);
    else launch_wide_g<D, KB, kWideRows>(a, s);
    return hipGetLastError();
}

template <int D>
hipError_t launch_wide_d(const AttnArgs& a, hipStream_t s) {
    switch (a.kc.bits) {
        case 1: return launch_wide_k<D, 1>(a, s);
        case 2: return launch_wide_k<D, 2>(a, s);
        case 3: return launch_wide_k<D, 3>(a, s);
        default: return launch_wide_k<D, 4>(a, s);
    }
}

}  // namespace

// d = 512 runs on the matrix cores (tq_attn_wide_mc.hip); this kernel serves
// d = 256 caches with two norm blocks
hipError_t launch_wide(const AttnArgs& a, hipStream_t s) {
    return a.kc.d == 512 ? launch_wide_mc(a, s) : launch_wide_d<256>(a, s);
}

}  // namespace tqi
