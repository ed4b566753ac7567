// Host side of decode attention: launch planning, workspace layout and the
// launches (QJL query projection when the keys carry QJL bits, split-K scan,
// combine + inverse transform, or with a residual window the window kernel,
// which also combines).
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <atomic>

#include "tq_attn_kernels.h"
#include "tq_internal.h"

namespace tqi {

// Resident split blocks per compute unit for this variant (cached).
static int split_blocks_any(int d, int kb, int vb, bool qjl) {
    static std::atomic<int> cache[3][4][4][2];
    std::atomic<int>& c = cache[d == 64 ? 2 : (d == 128 ? 0 : 1)][kb - 1][vb - 1][qjl ? 1 : 0];
    int nb = c.load(std::memory_order_relaxed);
    if (nb > 0) return nb;
    if (d == 64) {
        nb = kb == 2 ? split_blocks_dk<64, 2>(vb, qjl) : split_blocks_dk<64, 4>(vb, qjl);
    } else if (d == 128) {
        switch (kb) {
            case 1: nb = split_blocks_dk<128, 1>(vb, qjl); break;
            case 2: nb = split_blocks_dk<128, 2>(vb, qjl); break;
            case 3: nb = split_blocks_dk<128, 3>(vb, qjl); break;
            default: nb = split_blocks_dk<128, 4>(vb, qjl); break;
        }
    } else {
        switch (kb) {
            case 1: nb = split_blocks_dk<256, 1>(vb, qjl); break;
            case 2: nb = split_blocks_dk<256, 2>(vb, qjl); break;
            case 3: nb = split_blocks_dk<256, 3>(vb, qjl); break;
            default: nb = split_blocks_dk<256, 4>(vb, qjl); break;
        }
    }
    if (nb <= 0) return 1;  // occupancy unknown (no device): not cached
    c.store(nb, std::memory_order_relaxed);
    return nb;
}

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>* c = dev < 64 ? &cache[dev] : nullptr;
    int n = c ? c->load(std::memory_order_relaxed) : 0;
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 1;
    if (c) c->store(n, std::memory_order_relaxed);
    return n;
}

// The query rows of one kv head (g heads in each of the ncols query columns,
// gv = g * ncols rows) are processed in chunks of G rows, the largest divisor
// of gv not above 16 where the scan has 16-row blocks (no QJL, d <= 128), else
// not above 8.  The context is cut into splits of a
// multiple of 64 tokens.  With S resident block slots on the device (compute
// units x blocks per unit for this variant), a grid of B blocks runs in
// ceil(B / S) rounds and a block costs about (tiles per wave + 2) tile times
// (the 2 covers its table setup and merge); the split count minimising
// rounds x block cost is taken, among the largest split counts that fit 1..8
// rounds.  The plan depends on the current device.
void attn_plan(int batch, int hkv, int gv, int64_t ctx_cap, int d, int kb, int vb, bool qjl, int* splits,
               int64_t* split_tokens, int* heads_per_chunk) {
    int G = 1;
    for (int c = attn::split_rows16(d, qjl) ? 16 : 8; c >= 1; --c) {
        if (gv % c == 0) {
            G = c;
            break;
        }
    }
    *heads_per_chunk = G;
    const int64_t units = (int64_t)batch * hkv * (gv / G);
    const int64_t slots = (int64_t)device_cus() * split_blocks_any(d, kb, vb, qjl);
    const int64_t max_splits = ctx_cap > 0 ? (ctx_cap + 63) / 64 : 1;
    int64_t best_sp = 1, best_per = ((ctx_cap > 0 ? ctx_cap : 1) + 63) & ~(int64_t)63;
    double best_cost = -1.0;
    for (int r = 1; r <= 8; ++r) {
        int64_t sp = r * slots / units;
        if (sp < 1) sp = 1;
        if (sp > max_splits) sp = max_splits;
        int64_t per = ctx_cap > 0 ? (ctx_cap + sp - 1) / sp : 64;
        per = (per + 63) & ~(int64_t)63;
        sp = ctx_cap > 0 ? (ctx_cap + per - 1) / per : 1;
        const int64_t rounds = (units * sp + slots - 1) / slots;
        const int64_t nw = attn::split_waves(d, kb, vb, qjl);
        const int64_t wave_tiles = (per / 64 + nw - 1) / nw;
        const double cost = (double)rounds * (double)(wave_tiles + 2);
        if (best_cost < 0.0 || cost < best_cost || (cost == best_cost && sp < best_sp)) {
            best_cost = cost;
            best_sp = sp;
            best_per = per;
        }
    }
    // A positive TQ_ATTN_SPLITS in the environment replaces the chosen split
    // count (clamped to [1, 64-token tiles of the capacity]); tests use it to
    // check that the result does not depend on the split.  Read per call, so
    // the workspace query and the call that follows agree.
    if (const char* env = getenv("TQ_ATTN_SPLITS")) {
        const long want = strtol(env, nullptr, 10);
        if (want > 0 && ctx_cap > 0) {
            int64_t sp = want < max_splits ? (int64_t)want : max_splits;
            int64_t per = ((ctx_cap + sp - 1) / sp + 63) & ~(int64_t)63;
            best_per = per;
            best_sp = (ctx_cap + per - 1) / per;
        }
    }
    *splits = (int)best_sp;
    *split_tokens = best_per;
}

bool attn_wide(int d) { return d == 512; }

// Plan of the wide kernels: query rows in chunks of G <= 8 (the largest divisor of g);
// splits of a multiple of 256 tokens (4 waves x 64), as many as give about two
// blocks per compute unit (its registers and LDS hold two).
void wide_plan(int batch, int hkv, int g, int64_t ctx_cap, int* splits, int64_t* split_tokens, int* heads_per_chunk) {
    int G = 1;
    for (int c = 8; c >= 1; --c) {
        if (g % c == 0) {
            G = c;
            break;
        }
    }
    *heads_per_chunk = G;
    const int64_t units = (int64_t)batch * hkv * (g / G);
    const int64_t max_splits = ctx_cap > 0 ? (ctx_cap + 255) / 256 : 1;
    int64_t sp = (2 * (int64_t)device_cus() + units - 1) / units;
    sp = sp < 1 ? 1 : (sp > max_splits ? max_splits : sp);
    int64_t per = ctx_cap > 0 ? (ctx_cap + sp - 1) / sp : 256;
    per = (per + 255) & ~(int64_t)255;
    if (const char* env = getenv("TQ_ATTN_SPLITS")) {  // test hook, as for the scan
        const long want = strtol(env, nullptr, 10);
        if (want > 0 && ctx_cap > 0) {
            const int64_t w = want < max_splits ? (int64_t)want : max_splits;
            per = ((ctx_cap + w - 1) / w + 255) & ~(int64_t)255;
        }
    }
    sp = ctx_cap > 0 ? (ctx_cap + per - 1) / per : 1;
    *splits = (int)sp;
    *split_tokens = per;
}

static size_t align_floats(size_t n) { return (n + 63) & ~(size_t)63; }

size_t attn_workspace(int batch, int hq, int d, int m, int splits) {
    const size_t heads = (size_t)batch * hq;
    const size_t floats = align_floats(heads * (size_t)m) + align_floats(heads * (size_t)splits * (d + 2));
    return floats * sizeof(float);
}

template <int D>
static hipError_t launch_qprep_combine(const AttnArgs& a, hipStream_t s, bool prep) {
    if (prep) {
        constexpr int VPW = 64 / (D / 8);
        const int heads = a.batch * a.ncols * a.hq;
        const int grid = (heads + VPW - 1) / VPW;
        switch (a.q_dtype) {
            case TQ_F32: hipLaunchKernelGGL((attn::qprep_kernel<D, 0>), dim3(grid), dim3(64), 0, s, a); break;
            case TQ_F16: hipLaunchKernelGGL((attn::qprep_kernel<D, 1>), dim3(grid), dim3(64), 0, s, a); break;
            default: hipLaunchKernelGGL((attn::qprep_kernel<D, 2>), dim3(grid), dim3(64), 0, s, a); break;
        }
    } else {
        constexpr int HPB = 256 / (D / 8);  // heads per combine block
        hipLaunchKernelGGL((attn::combine_kernel<D>), dim3((a.batch * a.ncols * a.hq + HPB - 1) / HPB), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <int D>
static void launch_window(const AttnArgs& a, int grid, hipStream_t s) {
    switch (a.win_dtype) {
        case TQ_F32: hipLaunchKernelGGL((attn::window_kernel<D, 0>), dim3(grid), dim3(256), 0, s, a); break;
        case TQ_F16: hipLaunchKernelGGL((attn::window_kernel<D, 1>), dim3(grid), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((attn::window_kernel<D, 2>), dim3(grid), dim3(256), 0, s, a); break;
    }
}

static hipError_t launch_split_any(const AttnArgs& a, hipStream_t s) {
    if (a.kc.d == 64) return a.kc.bits == 2 ? launch_split_dk<64, 2>(a, s) : launch_split_dk<64, 4>(a, s);
    if (a.kc.d == 128) {
        switch (a.kc.bits) {
            case 1: return launch_split_dk<128, 1>(a, s);
            case 2: return launch_split_dk<128, 2>(a, s);
            case 3: return launch_split_dk<128, 3>(a, s);
            default: return launch_split_dk<128, 4>(a, s);
        }
    }
    switch (a.kc.bits) {
        case 1: return launch_split_dk<256, 1>(a, s);
        case 2: return launch_split_dk<256, 2>(a, s);
        case 3: return launch_split_dk<256, 3>(a, s);
        default: return launch_split_dk<256, 4>(a, s);
    }
}

static hipError_t launch_qprep_combine_any(const AttnArgs& a, hipStream_t s, bool prep) {
    switch (a.kc.d) {
        case 64: return launch_qprep_combine<64>(a, s, prep);
        case 128: return launch_qprep_combine<128>(a, s, prep);
        case 256: return launch_qprep_combine<256>(a, s, prep);
        default: {
            // d = 512 (no residual, so nothing to prepare): the combine only
            if (prep) return hipSuccess;
            constexpr int HPB = 256 / 64;
            hipLaunchKernelGGL((attn::combine_kernel<512>), dim3((a.batch * a.ncols * a.hq + HPB - 1) / HPB),
                               dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
}

hipError_t launch_attn(const AttnArgs& a, int stages, hipStream_t s) {
    hipError_t e = hipSuccess;
    // without QJL the scan rotates its queries itself and there is nothing to prepare
    if ((stages & ATTN_PREPARE) && a.kc.qjl_m > 0) {
        e = launch_qprep_combine_any(a, s, true);
        if (e != hipSuccess) return e;
    }
    if (stages & ATTN_SCAN) {
        e = attn_wide(a.kc.d) ? launch_wide(a, s) : launch_split_any(a, s);
        if (e != hipSuccess) return e;
    }
    if ((stages & ATTN_WINDOW) && a.win_cap > 0) {
        // the window kernel also merges the splits and writes the output:
        // one block per (batch, query head), heads of one kv head on one XCD
        const int grid = ((a.batch * a.hkv + 7) & ~7) * a.g;
        switch (a.kc.d) {
            case 64: launch_window<64>(a, grid, s); break;
            case 128: launch_window<128>(a, grid, s); break;
            default: launch_window<256>(a, grid, s); break;
        }
        return hipGetLastError();
    }
    if (stages & ATTN_COMBINE) e = launch_qprep_combine_any(a, s, false);
    return e;
}

}  // namespace tqi
