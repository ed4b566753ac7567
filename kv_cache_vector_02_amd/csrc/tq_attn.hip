// Host side of decode attention: launch planning, workspace layout and the
// three launches (query prep, split-K scan, combine + inverse transform).
#include <hip/hip_runtime.h>

#include "tq_attn_kernels.h"
#include "tq_internal.h"

namespace tqi {

// Query heads of one kv group are processed in chunks of G <= 8 heads (the
// largest divisor of g not above 8); splits cut the context so that roughly
// 1024 blocks of 256 threads cover the GPU, each split a multiple of 64 tokens
// and at least 256 tokens (one tile per wave).
void attn_plan(int batch, int hkv, int g, int64_t ctx_cap, int* splits, int64_t* split_tokens,
               int* heads_per_chunk) {
    int G = 1;
    for (int c = 8; c >= 1; --c) {
        if (g % c == 0) {
            G = c;
            break;
        }
    }
    const int64_t units = (int64_t)batch * hkv * (g / G);
    const int64_t target = 1024;
    const int64_t max_splits = ctx_cap > 0 ? (ctx_cap + 255) / 256 : 1;
    int64_t sp = (target + units - 1) / units;
    if (sp > max_splits) sp = max_splits;
    if (sp < 1) sp = 1;
    int64_t per = ctx_cap > 0 ? (ctx_cap + sp - 1) / sp : 64;
    per = (per + 63) & ~(int64_t)63;
    sp = ctx_cap > 0 ? (ctx_cap + per - 1) / per : 1;
    *splits = (int)sp;
    *split_tokens = per;
    *heads_per_chunk = G;
}

static size_t align_floats(size_t n) { return (n + 63) & ~(size_t)63; }

size_t attn_workspace(int batch, int hq, int d, int m, int splits) {
    const size_t heads = (size_t)batch * hq;
    const size_t floats = align_floats(heads * d) + align_floats(heads * (size_t)m) +
                          align_floats(heads * (size_t)splits * (d + 2));
    return floats * sizeof(float);
}

template <int D>
static hipError_t launch_qprep_combine(const AttnArgs& a, hipStream_t s, bool prep) {
    if (prep) {
        constexpr int VPW = 64 / (D / 8);
        const int heads = a.batch * a.hq;
        const int grid = (heads + VPW - 1) / VPW;
        switch (a.q_dtype) {
            case TQ_F32: hipLaunchKernelGGL((attn::qprep_kernel<D, 0>), dim3(grid), dim3(64), 0, s, a); break;
            case TQ_F16: hipLaunchKernelGGL((attn::qprep_kernel<D, 1>), dim3(grid), dim3(64), 0, s, a); break;
            default: hipLaunchKernelGGL((attn::qprep_kernel<D, 2>), dim3(grid), dim3(64), 0, s, a); break;
        }
    } else {
        hipLaunchKernelGGL((attn::combine_kernel<D>), dim3(a.batch * a.hq), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

static hipError_t launch_split_any(const AttnArgs& a, hipStream_t s) {
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

hipError_t launch_attn(const AttnArgs& a, int stages, hipStream_t s) {
    const bool d128 = a.kc.d == 128;
    hipError_t e = hipSuccess;
    if (stages & ATTN_PREPARE) {
        e = d128 ? launch_qprep_combine<128>(a, s, true) : launch_qprep_combine<256>(a, s, true);
        if (e != hipSuccess) return e;
    }
    if (stages & ATTN_SCAN) {
        e = launch_split_any(a, s);
        if (e != hipSuccess) return e;
    }
    if (stages & ATTN_COMBINE) e = d128 ? launch_qprep_combine<128>(a, s, false) : launch_qprep_combine<256>(a, s, false);
    return e;
}

}  // namespace tqi
