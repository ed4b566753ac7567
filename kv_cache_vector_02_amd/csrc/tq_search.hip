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
// Launches: qprep (A, stored k-major [d+m][n_q]), scan (grid = DB chunks x 64-query tiles; 64x64
// tiles of est through LDS, 4x4 register tiles per thread, exact per-block
// top-k lists in LDS), merge (per query, exact top-k over the block lists,
// ordered by estimate descending then id ascending).
#include <hip/hip_runtime.h>
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqi {
namespace {

using namespace tqd;

constexpr int BQ = 64;     // queries per block
constexpr int BT = 64;     // database rows per tile
constexpr int KC = 32;     // K chunk
constexpr int KMAX = 32;   // largest k

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
    if (m > 0) {
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

template <int D, int BITS>
__global__ __launch_bounds__(256) void search_scan_kernel(SearchArgs a) {
    constexpr int RB = D * BITS / 8;  // code bytes per row
    const int m = a.c.qjl_m;
    const int KD = D + m;
    const int k = a.k;
    __shared__ __attribute__((aligned(16))) float As[KC][BQ];
    __shared__ __attribute__((aligned(16))) float Bs[KC][BT];
    __shared__ float Es[BQ][BT + 1];
    __shared__ float lst_s[BQ][KMAX];
    __shared__ int32_t lst_i[BQ][KMAX];
    __shared__ __attribute__((aligned(16))) uint32_t rcode[BT * RB / 4];
    __shared__ __attribute__((aligned(16))) uint32_t rbits[BT * 8];  // m <= 256 -> 8 dwords per row
    __shared__ float rn[BT], rg[BT];
    __shared__ float cent[16];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int q0 = blockIdx.y * BQ;
    const int64_t r_beg = (int64_t)blockIdx.x * a.block_rows;
    const int64_t r_end = (r_beg + a.block_rows < a.n_db) ? r_beg + a.block_rows : a.n_db;

    if (tid < 16) cent[tid] = a.c.centroid[tid];
    for (int e = tid; e < BQ * KMAX; e += 256) {
        lst_s[e / KMAX][e % KMAX] = -INFINITY;
        lst_i[e / KMAX][e % KMAX] = -1;
    }
    __syncthreads();

    for (int64_t t0 = r_beg; t0 < r_end; t0 += BT) {
        const int nt = (int)((r_end - t0) < BT ? (r_end - t0) : BT);
        // stage the row tile: codes, sign bits, norm, gamma
        for (int e = tid; e < BT * RB / 4; e += 256) {
            const int r = e / (RB / 4);
            rcode[e] = r < nt ? reinterpret_cast<const uint32_t*>(a.codes + (t0 + r) * RB)[e % (RB / 4)] : 0u;
        }
        if (m > 0) {
            const int mw = m >> 5;
            for (int e = tid; e < BT * mw; e += 256) {
                const int r = e / mw;
                rbits[r * 8 + e % mw] = r < nt ? reinterpret_cast<const uint32_t*>(a.qjl + (t0 + r) * (m >> 3))[e % mw] : 0u;
            }
        }
        if (tid < BT) {
            rn[tid] = tid < nt ? half_bits_to_float(a.norms[t0 + tid]) : 0.0f;
            rg[tid] = (tid < nt && m > 0) ? half_bits_to_float(a.gamma[t0 + tid]) : 0.0f;
        }
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

        for (int k0 = 0; k0 < KD; k0 += KC) {
            __syncthreads();
            // A chunk: As[kk][q] = A[q0+q][k0+kk] (A is stored k-major: [d+m][n_q])
            for (int e = tid; e < KC * BQ; e += 256) {
                const int kk = e / BQ, q = e % BQ;
                As[kk][q] = (q0 + q < a.n_q) ? a.qrot[(int64_t)(k0 + kk) * a.n_q + q0 + q] : 0.0f;
            }
            // B chunk: 8 consecutive k of one row per thread
            {
                const int r = tid >> 2, kb = (tid & 3) * 8;
                float vals[8];
                if (k0 < D) {
                    const int bit0 = (k0 + kb) * BITS;  // 8 codes = BITS bytes
                    const uint8_t* rp = reinterpret_cast<const uint8_t*>(rcode) + r * RB + bit0 / 8;
                    uint32_t packed = 0;
#pragma unroll
                    for (int x = 0; x < BITS; ++x) packed |= (uint32_t)rp[x] << (8 * x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[e] = cent[(packed >> (BITS * e)) & ((1u << BITS) - 1u)];
                } else {
                    const int j0 = k0 - D + kb;
                    const uint32_t w = rbits[r * 8 + (j0 >> 5)] >> (j0 & 31);
                    const float gm = rg[r];
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[e] = ((w >> e) & 1u) ? gm : -gm;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) Bs[kb + e][r] = vals[e];
            }
            __syncthreads();
#pragma unroll 8
            for (int kk = 0; kk < KC; ++kk) {
                const float4 av = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
                const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
                const float ar[4] = {av.x, av.y, av.z, av.w};
                const float br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = tx * 4 + j;
                Es[ty * 4 + i][t] = t < nt ? rn[t] * acc[i][j] : -INFINITY;
            }
        __syncthreads();
        // per-query insertion into the exact top-k list (score desc, id asc;
        // ids grow along the scan, so an equal score never displaces an entry)
        if (tid < BQ) {
            float* ls = lst_s[tid];
            int32_t* li = lst_i[tid];
            for (int t = 0; t < nt; ++t) {
                const float sc = Es[tid][t];
                if (sc > ls[k - 1]) {
                    int pos = k - 1;
                    while (pos > 0 && ls[pos - 1] < sc) {
                        ls[pos] = ls[pos - 1];
                        li[pos] = li[pos - 1];
                        --pos;
                    }
                    ls[pos] = sc;
                    li[pos] = (int32_t)(t0 + t);
                }
            }
        }
    }
    __syncthreads();
    // block candidates -> workspace [n_q][n_blocks][k]
    for (int e = tid; e < BQ * k; e += 256) {
        const int q = e / k, j = e % k;
        if (q0 + q < a.n_q) {
            const int64_t o = ((int64_t)(q0 + q) * a.n_blocks + blockIdx.x) * k + j;
            a.cand_s[o] = lst_s[q][j];
            a.cand_i[o] = lst_i[q][j];
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

template <int D>
hipError_t launch_scan_b(const SearchArgs& a, hipStream_t s) {
    const dim3 grid(a.n_blocks, (a.n_q + BQ - 1) / BQ);
    switch (a.c.bits) {
        case 1: hipLaunchKernelGGL((search_scan_kernel<D, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((search_scan_kernel<D, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((search_scan_kernel<D, 3>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((search_scan_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

void search_plan(int n_q, int64_t n_db, int k, int* n_blocks, int64_t* block_rows) {
    // DB chunks of a multiple of 64 rows, about 4096 rows, at most ~4096
    // candidates per query for the merge.
    (void)n_q;
    int64_t rows = 4096;
    int64_t nb = (n_db + rows - 1) / rows;
    const int64_t max_nb = 4096 / (k > 0 ? k : 1);
    if (nb > max_nb) {
        nb = max_nb;
        rows = ((n_db + nb - 1) / nb + 63) & ~(int64_t)63;
        nb = (n_db + rows - 1) / rows;
    }
    if (nb < 1) nb = 1;
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
