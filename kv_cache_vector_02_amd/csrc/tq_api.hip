// Host side of the C ABI declared in include/tq.h: codebook construction,
// argument validation, workspace sizing and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cmath>

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "tq.h"
#include "tq_internal.h"

namespace {

// ------------------------------------------------------------ codebook ----
double normal_pdf(double x) {
    if (isinf(x)) return 0.0;
    return exp(-0.5 * x * x) * 0.3989422804014327;  // 1/sqrt(2 pi)
}

// P(X > x) for X ~ N(0,1); erfc keeps the tail accurate.
double normal_tail(double x) {
    if (isinf(x)) return x > 0 ? 0.0 : 1.0;
    return 0.5 * erfc(x * 0.7071067811865476);
}

// x with P(X > x) = p, 0 < p <= 0.5, by bisection (x >= 0).
double tail_inverse(double p) {
    double lo = 0.0, hi = 40.0;
    for (int i = 0; i < 200; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (normal_tail(mid) > p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

// Lloyd-Max quantiser of N(0,1) with 2^bits levels: the fixed point of
// "centroid = conditional mean of its cell" and "threshold = midpoint of the
// neighbouring centroids", solved on the positive half (cells [tau_k, tau_k+1)
// with tau_0 = 0, tau_half = inf) and mirrored.
void lloyd_max(int bits, double* cent, double* thr) {
    const int L = 1 << bits, half = L / 2;
    double tau[9], c[8];
    tau[0] = 0.0;
    for (int k = 1; k < half; ++k) tau[k] = tail_inverse(0.5 - (double)k / L);
    tau[half] = INFINITY;
    for (int it = 0; it < 1000000; ++it) {
        for (int k = 0; k < half; ++k)
            c[k] = (normal_pdf(tau[k]) - normal_pdf(tau[k + 1])) / (normal_tail(tau[k]) - normal_tail(tau[k + 1]));
        double delta = 0.0;
        for (int k = 1; k < half; ++k) {
            const double nt = 0.5 * (c[k - 1] + c[k]);
            delta = fmax(delta, fabs(nt - tau[k]));
            tau[k] = nt;
        }
        if (delta < 1e-15) break;
    }
    for (int k = 0; k < half; ++k)
        c[k] = (normal_pdf(tau[k]) - normal_pdf(tau[k + 1])) / (normal_tail(tau[k]) - normal_tail(tau[k + 1]));
    for (int k = 0; k < half; ++k) {
        cent[half + k] = c[k];
        cent[half - 1 - k] = -c[k];
    }
    thr[half - 1] = 0.0;
    for (int k = 1; k < half; ++k) {
        const double t = 0.5 * (c[k - 1] + c[k]);
        thr[half - 1 + k] = t;
        thr[half - 1 - k] = -t;
    }
}

// SplitMix64 output number `index` (1-based) from state `seed`.
uint64_t splitmix64_at(uint64_t seed, uint64_t index) {
    uint64_t z = seed + index * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

bool valid_d(int d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }

bool valid_codec(const tq_codec* c) {
    if (!(c && valid_d(c->d) && c->bits >= 1 && c->bits <= 4 && c->qjl_m >= 0 && c->qjl_m <= 256 &&
          c->qjl_m % 32 == 0))
        return false;
    if (c->rotation != TQ_ROT_WHT && !(c->rotation == TQ_ROT_DOUBLE && c->d == 64)) return false;
    if (c->norm_blocks != 1 && !(c->norm_blocks == 2 && c->d >= 256 && c->residual == TQ_RES_NONE)) return false;
    if (c->d == 512 && c->residual != TQ_RES_NONE) return false;
    switch (c->residual) {
        case TQ_RES_NONE: return c->qjl_m == 0;
        case TQ_RES_QJL: return c->qjl_m > 0;
        case TQ_RES_SRHT:
        case TQ_RES_SIGN: return c->qjl_m == c->d;
        default: return false;
    }
}

// The residual needs the caller's Gaussian projection S.
bool needs_S(const tq_codec* c) { return c->residual == TQ_RES_QJL; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int finish(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EDEVICE; }

}  // namespace

namespace tqi {
// Bin table of the encoder's quantizer.  The index of z = w / n is the number
// of thresholds below it; with bins b = floor(z * s + off) that each hold at
// most one threshold, every value away from the bin edges needs the count
// below its bin and one compare with the bin's threshold.  The plan puts no
// threshold within 1/64 of a bin edge, far beyond the rounding of z * s + off
// in float32, so a value whose bin is misjudged lies away from any threshold
// and the count and compare still give its exact index.  Bins cover
// |z| <= sqrt(d) (the largest |w| / n) with margin; qt_n = 0 leaves the
// encoder to count the thresholds one by one.  The search starts at the
// smallest scale whose bins are narrower than the closest pair of thresholds,
// and plans are cached per (d, bits, thresholds): every call fills the
// launch arguments.
struct QtabPlan {
    float scale, off, inv_scale;
    int32_t n;
};

static QtabPlan search_qtab(int d, int nt, const float* th) {
    QtabPlan p{0.0f, 0.0f, 0.0f, 0};
    double gap = INFINITY;
    for (int j = 0; j < nt; ++j) {
        if (!std::isfinite(th[j]) || (j > 0 && !(th[j] > th[j - 1]))) return p;
        if (j > 0) gap = std::fmin(gap, (double)th[j] - (double)th[j - 1]);
    }
    const double zmax = std::sqrt((double)d) * 1.001 + 0.5;
    const double edge = 1.0 / 64.0;
    const int si0 = nt > 1 ? (int)std::ceil((1.0 / gap - 1.0) * 8.0) : 0;
    for (int si = si0 < 0 ? 0 : si0; si <= 504; ++si) {
        const double s = 1.0 + 0.125 * si;  // bins per unit of z, exact in float32
        for (int fi = 0; fi < 64; ++fi) {
            const double off = std::ceil(zmax * s) + 1.0 + fi / 64.0;
            const int nb = (int)std::floor(zmax * s + off) + 2;
            if (nb > kQTabMax) return p;  // larger scales need more bins still
            bool ok = true;
            double prev = -1.0;
            for (int j = 0; j < nt && ok; ++j) {
                const double x = (double)th[j] * s + off, b = std::floor(x), fr = x - b;
                ok = fr >= edge && fr <= 1.0 - edge && b > prev;
                prev = b;
            }
            if (ok) return QtabPlan{(float)s, (float)off, (float)(1.0 / s), nb};
        }
    }
    return p;
}

static void plan_qtab(const tq_codec* c, CodecArgs* a) {
    struct Entry {
        int d, bits;
        float th[15];
        QtabPlan plan;
    };
    static std::mutex mu;
    static Entry cache[16];
    static int used = 0, next = 0;
    const int nt = (1 << c->bits) - 1;
    QtabPlan plan;
    bool hit = false;
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < used && !hit; ++i) {
            const Entry& e = cache[i];
            if (e.d == c->d && e.bits == c->bits && memcmp(e.th, c->threshold, nt * sizeof(float)) == 0) {
                plan = e.plan;
                hit = true;
            }
        }
    }
    if (!hit) {
        plan = search_qtab(c->d, nt, c->threshold);
        std::lock_guard<std::mutex> g(mu);
        Entry& e = cache[next];
        e.d = c->d;
        e.bits = c->bits;
        memcpy(e.th, c->threshold, nt * sizeof(float));
        e.plan = plan;
        next = (next + 1) % 16;
        used = used < 16 ? used + 1 : 16;
    }
    a->qt_scale = plan.scale;
    a->qt_off = plan.off;
    a->qt_inv_scale = plan.inv_scale;
    a->qt_n = plan.n;
}

void fill_codec_args(const tq_codec* c, CodecArgs* a) {
    memcpy(a->sign_mask, c->sign_mask, sizeof(c->sign_mask));
    memcpy(a->sign_mask + 8, c->sign_mask_hi, sizeof(c->sign_mask_hi));
    memcpy(a->centroid, c->centroid, sizeof(a->centroid));
    memcpy(a->threshold, c->threshold, sizeof(a->threshold));
    a->d = c->d;
    a->bits = c->bits;
    a->qjl_m = c->qjl_m;
    a->residual = c->residual;
    memcpy(a->sign_mask2, c->sign_mask2, sizeof(a->sign_mask2));
    a->rotation = c->rotation;
    a->norm_blocks = c->norm_blocks;
    memcpy(a->sign_mask3, c->sign_mask3, sizeof(a->sign_mask3));
    plan_qtab(c, a);
}
}  // namespace tqi

extern "C" {

int tq_codebook_opts(int bits, int d, uint64_t seed, int residual, int qjl_m, int rotation, int norm_blocks,
                     tq_codec* out) {
    if (!out) return TQ_EINVAL;
    if (!valid_d(d) || bits < 1 || bits > 4 || qjl_m < 0 || qjl_m > 256 || qjl_m % 32 != 0)
        return TQ_EUNSUPPORTED;
    if (rotation != TQ_ROT_WHT && !(rotation == TQ_ROT_DOUBLE && d == 64)) return TQ_EUNSUPPORTED;
    if (norm_blocks != 1 && !(norm_blocks == 2 && d >= 256 && residual == TQ_RES_NONE)) return TQ_EUNSUPPORTED;
    if (d == 512 && residual != TQ_RES_NONE) return TQ_EUNSUPPORTED;
    if (residual == TQ_RES_SRHT || residual == TQ_RES_SIGN) {
        if (qjl_m != 0 && qjl_m != d) return TQ_EUNSUPPORTED;
        qjl_m = d;
    } else if (residual == TQ_RES_QJL) {
        if (qjl_m == 0) return TQ_EUNSUPPORTED;
    } else if (residual != TQ_RES_NONE || qjl_m != 0) {
        return TQ_EUNSUPPORTED;
    }
    memset(out, 0, sizeof(*out));
    out->d = d;
    out->bits = bits;
    out->qjl_m = qjl_m;
    out->residual = residual;
    out->seed = seed;
    out->rotation = rotation;
    out->norm_blocks = norm_blocks;
    for (int i = 0; i < d; ++i) {
        if (splitmix64_at(seed, (uint64_t)i + 1) >> 63) {
            if (i < 256) out->sign_mask[i >> 5] |= 1u << (i & 31);
            else out->sign_mask_hi[(i - 256) >> 5] |= 1u << (i & 31);
        }
        if (i >= 256) continue;
        // the second sign basis: outputs 257.. (1..256 belong to the first at d <= 256);
        // the double transform's second flip: outputs 513..
        if (splitmix64_at(seed, (uint64_t)i + 257) >> 63) out->sign_mask2[i >> 5] |= 1u << (i & 31);
        if (splitmix64_at(seed, (uint64_t)i + 513) >> 63) out->sign_mask3[i >> 5] |= 1u << (i & 31);
    }
    double c[16], t[15];
    lloyd_max(bits, c, t);
    const int L = 1 << bits;
    for (int k = 0; k < L; ++k) out->centroid[k] = (float)c[k];
    for (int k = 0; k < L - 1; ++k) out->threshold[k] = (float)t[k];
    return TQ_OK;
}

int tq_codebook_ex(int bits, int d, uint64_t seed, int residual, int qjl_m, tq_codec* out) {
    return tq_codebook_opts(bits, d, seed, residual, qjl_m, TQ_ROT_WHT, 1, out);
}

int tq_codebook(int bits, int d, uint64_t seed, int qjl_m, tq_codec* out) {
    return tq_codebook_ex(bits, d, seed, qjl_m > 0 ? TQ_RES_QJL : TQ_RES_NONE, qjl_m, out);
}

size_t tq_packed_bytes(int d, int bits, int qjl_m) {
    if (d <= 0 || bits < 1 || bits > 4 || qjl_m < 0) return 0;
    size_t n = (size_t)d * bits / 8 + 2;
    if (qjl_m) n += (size_t)qjl_m / 8 + 2;
    return n;
}

const char* tq_strerror(int code) {
    switch (code) {
        case TQ_OK: return "ok";
        case TQ_EINVAL: return "invalid argument (null pointer, size, stride or alignment)";
        case TQ_EUNSUPPORTED: return "unsupported configuration (d, bits, qjl_m, k or head ratio)";
        case TQ_EWORKSPACE: return "workspace missing or too small";
        case TQ_EDEVICE: return "HIP launch failed";
        case TQ_ESCRATCH: return "request exceeds the static scratch of the no-alloc entry point";
        default: return "unknown error code";
    }
}

// Validates one encode job and fills its launch arguments (nothing is launched).
static int encode_setup(const tq_codec* c, const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
                        uint8_t* codes, int64_t code_row_stride, uint16_t* norms_f16, const float* qjl_S,
                        uint8_t* qjl_bits, uint16_t* qjl_gamma_f16, tqi::EncodeArgs* a) {
    if (!c) return TQ_EINVAL;
    if (!valid_codec(c)) return TQ_EUNSUPPORTED;
    if (x_dtype != TQ_F32 && x_dtype != TQ_F16 && x_dtype != TQ_BF16) return TQ_EINVAL;
    if (n < 0) return TQ_EINVAL;
    const int esz = x_dtype == TQ_F32 ? 4 : 2;
    if (n > 0) {
        if (!x || !codes || !norms_f16 || !aligned(x, 16) || !aligned(codes, 4) || !aligned(norms_f16, 2))
            return TQ_EINVAL;
        if (x_row_stride < c->d || (x_row_stride * esz) % 16 != 0) return TQ_EINVAL;
        if (code_row_stride < c->d * c->bits / 8 || code_row_stride % 4 != 0) return TQ_EINVAL;
        if (c->qjl_m > 0) {
            if (!qjl_bits || !qjl_gamma_f16 || !aligned(qjl_bits, 4) || !aligned(qjl_gamma_f16, 2)) return TQ_EINVAL;
            if (needs_S(c) && (!qjl_S || !aligned(qjl_S, 16))) return TQ_EINVAL;
        }
    }
    tqi::fill_codec_args(c, &a->c);
    a->x = x;
    a->n = n;
    a->x_stride = x_row_stride;
    a->codes = codes;
    a->code_stride = code_row_stride;
    a->norms = norms_f16;
    a->S = qjl_S;
    a->qjl = qjl_bits;
    a->gamma = qjl_gamma_f16;
    a->pos = nullptr;
    a->cap = 0;
    a->seq_heads = 1;
    a->grp_rows = 0;
    a->grp_off = 0;
    return TQ_OK;
}

int tq_encode(const tq_codec* c, const void* x, int x_dtype, int64_t n, int64_t x_row_stride, uint8_t* codes,
              int64_t code_row_stride, uint16_t* norms_f16, const float* qjl_S, uint8_t* qjl_bits,
              uint16_t* qjl_gamma_f16, void* stream) {
    tqi::EncodeArgs a;
    const int rc = encode_setup(c, x, x_dtype, n, x_row_stride, codes, code_row_stride, norms_f16, qjl_S, qjl_bits,
                                qjl_gamma_f16, &a);
    if (rc != TQ_OK || n == 0) return rc;
    return finish(tqi::launch_encode(a, x_dtype, (hipStream_t)stream));
}

int tq_encode_kv(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v, int x_dtype, int64_t n,
                 int64_t x_row_stride, uint8_t* k_codes, int64_t k_code_row_stride, uint16_t* k_norms_f16,
                 uint8_t* v_codes, int64_t v_code_row_stride, uint16_t* v_norms_f16, const float* qjl_S,
                 uint8_t* k_qjl_bits, uint16_t* k_qjl_gamma_f16, void* stream) {
    if (!kc || !vc) return TQ_EINVAL;
    if (kc->d != vc->d || vc->qjl_m != 0) return TQ_EUNSUPPORTED;
    tqi::EncodeArgs ka, va;
    int rc = encode_setup(kc, k, x_dtype, n, x_row_stride, k_codes, k_code_row_stride, k_norms_f16, qjl_S, k_qjl_bits,
                          k_qjl_gamma_f16, &ka);
    if (rc == TQ_OK)
        rc = encode_setup(vc, v, x_dtype, n, x_row_stride, v_codes, v_code_row_stride, v_norms_f16, nullptr, nullptr,
                          nullptr, &va);
    if (rc != TQ_OK || n == 0) return rc;
    return finish(tqi::launch_encode_pair(ka, va, x_dtype, (hipStream_t)stream));
}

int tq_prefill(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v, int x_dtype, int n_heads,
               int64_t tokens, int64_t t0, int64_t ctx_cap, uint8_t* k_codes, uint16_t* k_norms_f16, uint8_t* v_codes,
               uint16_t* v_norms_f16, const float* qjl_S, uint8_t* k_qjl_bits, uint16_t* k_qjl_gamma_f16,
               void* stream) {
    if (!kc || !vc) return TQ_EINVAL;
    if (kc->d != vc->d || vc->qjl_m != 0) return TQ_EUNSUPPORTED;
    if (n_heads <= 0 || tokens < 0 || t0 < 0 || ctx_cap <= 0 || t0 + tokens > ctx_cap) return TQ_EINVAL;
    const int64_t n = (int64_t)n_heads * tokens;
    tqi::EncodeArgs ka, va;
    // cache rows are exactly d*bits/8 bytes (the layout the attention calls read)
    int rc = encode_setup(kc, k, x_dtype, n, kc->d, k_codes, kc->d * kc->bits / 8, k_norms_f16, qjl_S, k_qjl_bits,
                          k_qjl_gamma_f16, &ka);
    if (rc == TQ_OK)
        rc = encode_setup(vc, v, x_dtype, n, vc->d, v_codes, vc->d * vc->bits / 8, v_norms_f16, nullptr, nullptr,
                          nullptr, &va);
    if (rc != TQ_OK || n == 0) return rc;
    for (tqi::EncodeArgs* a : {&ka, &va}) {
        a->cap = ctx_cap;
        a->grp_rows = tokens;
        a->grp_off = t0;
    }
    return finish(tqi::launch_encode_pair(ka, va, x_dtype, (hipStream_t)stream));
}

int tq_append(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v, int x_dtype, int batch,
              int n_heads, const int32_t* pos, int64_t ctx_cap, uint8_t* k_codes, uint16_t* k_norms_f16,
              uint8_t* v_codes, uint16_t* v_norms_f16, const float* qjl_S, uint8_t* k_qjl_bits,
              uint16_t* k_qjl_gamma_f16, void* stream) {
    if (!kc || !vc) return TQ_EINVAL;
    if (kc->d != vc->d || vc->qjl_m != 0) return TQ_EUNSUPPORTED;
    if (batch <= 0 || n_heads <= 0 || ctx_cap <= 0 || !pos || !aligned(pos, 4)) return TQ_EINVAL;
    const int64_t n = (int64_t)batch * n_heads;
    tqi::EncodeArgs ka, va;
    // cache rows are exactly d*bits/8 bytes (the layout the attention calls read)
    int rc = encode_setup(kc, k, x_dtype, n, kc->d, k_codes, kc->d * kc->bits / 8, k_norms_f16, qjl_S, k_qjl_bits,
                          k_qjl_gamma_f16, &ka);
    if (rc == TQ_OK)
        rc = encode_setup(vc, v, x_dtype, n, vc->d, v_codes, vc->d * vc->bits / 8, v_norms_f16, nullptr, nullptr,
                          nullptr, &va);
    if (rc != TQ_OK) return rc;
    for (tqi::EncodeArgs* a : {&ka, &va}) {
        a->pos = pos;
        a->cap = ctx_cap;
        a->seq_heads = n_heads;
    }
    return finish(tqi::launch_encode_pair(ka, va, x_dtype, (hipStream_t)stream));
}

int tq_decode(const tq_codec* c, const uint8_t* codes, int64_t code_row_stride, const uint16_t* norms_f16,
              int64_t n, float* x_hat, void* stream) {
    if (!c) return TQ_EINVAL;
    if (!valid_codec(c)) return TQ_EUNSUPPORTED;
    if (n < 0) return TQ_EINVAL;
    if (n == 0) return TQ_OK;
    if (!codes || !norms_f16 || !x_hat || !aligned(x_hat, 16) || !aligned(norms_f16, 2)) return TQ_EINVAL;
    if (code_row_stride < c->d * c->bits / 8) return TQ_EINVAL;
    tqi::DecodeArgs a;
    tqi::fill_codec_args(c, &a.c);
    a.codes = codes;
    a.code_stride = code_row_stride;
    a.norms = norms_f16;
    a.n = n;
    a.out = x_hat;
    return finish(tqi::launch_decode(a, (hipStream_t)stream));
}

static int attn_check(const tq_codec* kc, const tq_codec* vc, int batch, int ncols, int n_q_heads, int n_kv_heads,
                      int64_t ctx_cap, int* splits, int64_t* split_tokens, int* G) {
    if (!kc || !vc) return TQ_EINVAL;
    if (!valid_codec(kc) || !valid_codec(vc)) return TQ_EUNSUPPORTED;
    if (kc->d != vc->d || vc->qjl_m != 0) return TQ_EUNSUPPORTED;
    const bool wide = tqi::attn_wide(kc->d);
    if (wide) {
        // d = 512: the wide kernel, one query column, keys without a residual
        if (kc->qjl_m != 0 || ncols != 1) return TQ_EUNSUPPORTED;
    } else if (kc->d == 64) {
        // the scan's lane layout: key bytes a whole number of dwords per lane
        // group (2 or 4 bits) and 2..4-bit values
        if ((kc->bits != 2 && kc->bits != 4) || vc->bits < 2) return TQ_EUNSUPPORTED;
    } else if (kc->d != 128 && kc->d != 256) {
        return TQ_EUNSUPPORTED;
    }
    if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || ctx_cap <= 0 || batch > 65535 || ncols <= 0)
        return TQ_EINVAL;
    if (n_q_heads % n_kv_heads != 0 || ncols > TQ_MAX_QUERY_COLS) return TQ_EUNSUPPORTED;
    // one (batch, kv head) plane of any cache array must be addressable with 31-bit offsets
    const int64_t row_max = kc->d * (kc->bits > vc->bits ? kc->bits : vc->bits) / 8 + kc->qjl_m / 8;
    if (ctx_cap > (((int64_t)1 << 31) - 1) / (row_max > 2 ? row_max : 2)) return TQ_EUNSUPPORTED;
    const int gv = n_q_heads / n_kv_heads * ncols;  // query rows per kv head
    if (wide) tqi::wide_plan(batch, n_kv_heads, gv, ctx_cap, splits, split_tokens, G);
    else tqi::attn_plan(batch, n_kv_heads, gv, ctx_cap, kc->d, kc->bits, vc->bits, kc->qjl_m > 0, splits, split_tokens, G);
    if ((int64_t)n_kv_heads * (gv / *G) > 65535) return TQ_EUNSUPPORTED;
    return TQ_OK;
}

static size_t attn_ws_bytes(const tq_codec* kc, const tq_codec* vc, int batch, int ncols, int n_q_heads,
                            int n_kv_heads, int64_t ctx_cap) {
    int splits, G;
    int64_t per;
    if (attn_check(kc, vc, batch, ncols, n_q_heads, n_kv_heads, ctx_cap, &splits, &per, &G) != TQ_OK) return 0;
    return tqi::attn_workspace(batch * ncols, n_q_heads, kc->d, kc->qjl_m, splits);
}

size_t tq_attn_workspace_bytes(const tq_codec* kc, const tq_codec* vc, int batch, int n_q_heads, int n_kv_heads,
                               int64_t ctx_cap) {
    return attn_ws_bytes(kc, vc, batch, 1, n_q_heads, n_kv_heads, ctx_cap);
}

// Validates every argument of the decode-attention entry points and fills the
// launch description; nothing is launched here.
static int attn_setup(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch, int ncols,
                      int n_q_heads, int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap,
                      const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl, const uint16_t* k_gamma,
                      const float* qjl_S, const uint8_t* v_codes, const uint16_t* v_norms, const void* k_win,
                      const void* v_win, int win_dtype, const int32_t* win_len, int win_cap, float scale, float* out,
                      void* workspace, size_t workspace_bytes, tqi::AttnArgs* a, const tq_attn_opts* opts = nullptr) {
    int splits, G;
    int64_t per;
    const int rc = attn_check(kc, vc, batch, ncols, n_q_heads, n_kv_heads, ctx_cap, &splits, &per, &G);
    if (rc != TQ_OK) return rc;
    if (ncols > 1 && win_cap > 0) return TQ_EUNSUPPORTED;  // the residual window serves one query column
    if (tqi::attn_wide(kc->d)) {
        // the d = 512 kernel: no residual window and no softmax switches
        if (win_cap > 0) return TQ_EUNSUPPORTED;
        if (opts && (opts->score_mode != TQ_SCORE_PLAIN || opts->sparse_v > 0.0f)) return TQ_EUNSUPPORTED;
    }
    if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_EINVAL;
    if (!q || !ctx_len || !k_codes || !k_norms || !v_codes || !v_norms || !out) return TQ_EINVAL;
    if (!aligned(q, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(out, 16) ||
        !aligned(k_norms, 2) || !aligned(v_norms, 2) || !aligned(ctx_len, 4))
        return TQ_EINVAL;
    if (kc->qjl_m > 0 && (!k_qjl || !k_gamma || (needs_S(kc) && !qjl_S) || !aligned(k_qjl, 4) ||
                          !aligned(k_gamma, 2)))
        return TQ_EINVAL;
    if (!isfinite(scale)) return TQ_EINVAL;
    if (opts) {
        if (opts->score_mode < TQ_SCORE_PLAIN || opts->score_mode > TQ_SCORE_SOFTEN) return TQ_EINVAL;
        if (opts->score_mode != TQ_SCORE_PLAIN && !(isfinite(opts->sqnr) && opts->sqnr > 0.0f)) return TQ_EINVAL;
        if (opts->ref_tokens != 0 && opts->ref_tokens < 2) return TQ_EINVAL;
        if (!(opts->sparse_v >= 0.0f && opts->sparse_v <= 1.0f)) return TQ_EINVAL;
        if (win_cap > 0 && (opts->score_mode != TQ_SCORE_PLAIN || opts->sparse_v > 0.0f)) return TQ_EUNSUPPORTED;
    }
    if (win_cap < 0) return TQ_EINVAL;
    if (win_cap > 0) {
        if (win_dtype != TQ_F32 && win_dtype != TQ_F16 && win_dtype != TQ_BF16) return TQ_EINVAL;
        if (!k_win || !v_win || !win_len || !aligned(k_win, 16) || !aligned(v_win, 16) || !aligned(win_len, 4))
            return TQ_EINVAL;
    }
    const int d = kc->d, m = kc->qjl_m;
    const size_t need = tqi::attn_workspace(batch * ncols, n_q_heads, d, m, splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return TQ_EWORKSPACE;

    tqi::fill_codec_args(kc, &a->kc);
    tqi::fill_codec_args(vc, &a->vc);
    a->q = q;
    a->q_dtype = q_dtype;
    a->batch = batch;
    a->hq = n_q_heads;
    a->hkv = n_kv_heads;
    a->g = n_q_heads / n_kv_heads;
    a->ncols = ncols;
    a->heads_per_chunk = G;
    a->chunks = a->g * ncols / G;
    a->ctx_len = ctx_len;
    a->ctx_cap = ctx_cap;
    a->k_codes = k_codes;
    a->k_norms = k_norms;
    a->k_qjl = k_qjl;
    a->k_gamma = k_gamma;
    a->S = qjl_S;
    a->v_codes = v_codes;
    a->v_norms = v_norms;
    a->scale = scale;
    a->score_mode = opts ? opts->score_mode : TQ_SCORE_PLAIN;
    a->sqnr = opts ? opts->sqnr : 1.0f;
    {
        const double n0 = opts && opts->ref_tokens ? opts->ref_tokens : 2048.0;
        a->inv_ln_n0 = (float)(1.0 / log(n0));
        a->sharp_c = (float)(1.0 / (2.0 * (double)a->sqnr * sqrt(log(n0))));
    }
    a->sparse_log2 = opts && opts->sparse_v > 0.0f ? (float)log2((double)opts->sparse_v) : -INFINITY;
    a->out = out;
    const size_t heads = (size_t)batch * ncols * n_q_heads;
    float* ws = (float*)workspace;
    auto al = [](size_t n) { return (n + 63) & ~(size_t)63; };
    a->qproj = ws;
    a->part = ws + al(heads * (size_t)m);
    a->splits = splits;
    a->split_tokens = per;
    a->k_win = k_win;
    a->v_win = v_win;
    a->win_dtype = win_dtype;
    a->win_len = win_len;
    a->win_cap = win_cap;
    return TQ_OK;
}

#define TQ_ATTN_ENTRY(NAME, STAGE)                                                                            \
    int NAME(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch, int n_q_heads,     \
             int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap, const uint8_t* k_codes,                 \
             const uint16_t* k_norms, const uint8_t* k_qjl, const uint16_t* k_gamma, const float* qjl_S,       \
             const uint8_t* v_codes, const uint16_t* v_norms, float scale, float* out, void* workspace,        \
             size_t workspace_bytes, void* stream) {                                                          \
        tqi::AttnArgs a;                                                                                      \
        const int rc = attn_setup(kc, vc, q, q_dtype, batch, 1, n_q_heads, n_kv_heads, ctx_len, ctx_cap, k_codes, \
                                  k_norms, k_qjl, k_gamma, qjl_S, v_codes, v_norms, nullptr, nullptr, 0,       \
                                  nullptr, 0, scale, out, workspace, workspace_bytes, &a);                   \
        if (rc != TQ_OK) return rc;                                                                           \
        return finish(tqi::launch_attn(a, STAGE, (hipStream_t)stream));                                      \
    }

TQ_ATTN_ENTRY(tq_attn_decode, tqi::ATTN_ALL)
TQ_ATTN_ENTRY(tq_attn_prepare, tqi::ATTN_PREPARE)
TQ_ATTN_ENTRY(tq_attn_scan, tqi::ATTN_SCAN)
TQ_ATTN_ENTRY(tq_attn_combine, tqi::ATTN_COMBINE)

// Scratch of tq_attn_decode_noalloc: a static device array (one copy per
// device the library runs on), holding the split partials and QJL query
// projections between the launches of one call.  In host code `scratch` names
// a host-side stand-in, not the device array: only the address from
// hipGetSymbolAddress, taken once per device with that device current, is
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (nullptr on failure).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        g_scratch_ptr[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}
}  // namespace

int tq_attn_decode_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch,
                           int n_q_heads, int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap,
                           const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl,
                           const uint16_t* k_gamma, const float* qjl_S, const uint8_t* v_codes,
                           const uint16_t* v_norms, float scale, float* out, void* stream) {
    const size_t need = tq_attn_workspace_bytes(kc, vc, batch, n_q_heads, n_kv_heads, ctx_cap);
    if (need > TQ_NOALLOC_SCRATCH_BYTES) return TQ_ESCRATCH;
    void* ws = need > 0 ? scratch_address() : nullptr;
    if (need > 0 && !ws) return TQ_EDEVICE;
    // need == 0 means the sizes are invalid: attn_setup reports why
    tqi::AttnArgs a;
    const int rc = attn_setup(kc, vc, q, q_dtype, batch, 1, n_q_heads, n_kv_heads, ctx_len, ctx_cap, k_codes, k_norms,
                              k_qjl, k_gamma, qjl_S, v_codes, v_norms, nullptr, nullptr, 0, nullptr, 0, scale, out,
                              ws ? ws : (void*)nullptr, ws ? (size_t)TQ_NOALLOC_SCRATCH_BYTES : 0, &a);
    if (rc != TQ_OK) return rc;
    return finish(tqi::launch_attn(a, tqi::ATTN_ALL, (hipStream_t)stream));
}

int tq_attn_decode_rw(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch, int n_q_heads,
                      int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap, const uint8_t* k_codes,
                      const uint16_t* k_norms, const uint8_t* k_qjl, const uint16_t* k_gamma, const float* qjl_S,
                      const uint8_t* v_codes, const uint16_t* v_norms, const void* k_win, const void* v_win,
                      int win_dtype, const int32_t* win_len, int win_cap, float scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    tqi::AttnArgs a;
    const int rc = attn_setup(kc, vc, q, q_dtype, batch, 1, n_q_heads, n_kv_heads, ctx_len, ctx_cap, k_codes, k_norms,
                              k_qjl, k_gamma, qjl_S, v_codes, v_norms, k_win, v_win, win_dtype, win_len, win_cap,
                              scale, out, workspace, workspace_bytes, &a);
    if (rc != TQ_OK) return rc;
    return finish(tqi::launch_attn(a, tqi::ATTN_ALL | tqi::ATTN_WINDOW, (hipStream_t)stream));
}

int tq_attn_decode_ex(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch, int n_cols,
                      int n_q_heads, int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap, const uint8_t* k_codes,
                      const uint16_t* k_norms, const uint8_t* k_qjl, const uint16_t* k_gamma, const float* qjl_S,
                      const uint8_t* v_codes, const uint16_t* v_norms, float scale, const tq_attn_opts* opts,
                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
    tqi::AttnArgs a;
    const int rc = attn_setup(kc, vc, q, q_dtype, batch, n_cols, n_q_heads, n_kv_heads, ctx_len, ctx_cap, k_codes,
                              k_norms, k_qjl, k_gamma, qjl_S, v_codes, v_norms, nullptr, nullptr, 0, nullptr, 0, scale,
                              out, workspace, workspace_bytes, &a, opts);
    if (rc != TQ_OK) return rc;
    return finish(tqi::launch_attn(a, tqi::ATTN_ALL, (hipStream_t)stream));
}

int tq_attn_decode_mq(const tq_codec* kc, const tq_codec* vc, const void* q, int q_dtype, int batch, int n_cols,
                      int n_q_heads, int n_kv_heads, const int32_t* ctx_len, int64_t ctx_cap, const uint8_t* k_codes,
                      const uint16_t* k_norms, const uint8_t* k_qjl, const uint16_t* k_gamma, const float* qjl_S,
                      const uint8_t* v_codes, const uint16_t* v_norms, float scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    tqi::AttnArgs a;
    const int rc = attn_setup(kc, vc, q, q_dtype, batch, n_cols, n_q_heads, n_kv_heads, ctx_len, ctx_cap, k_codes,
                              k_norms, k_qjl, k_gamma, qjl_S, v_codes, v_norms, nullptr, nullptr, 0, nullptr, 0, scale,
                              out, workspace, workspace_bytes, &a);
    if (rc != TQ_OK) return rc;
    return finish(tqi::launch_attn(a, tqi::ATTN_ALL, (hipStream_t)stream));
}

static int search_check(const tq_codec* c, int n_q, int64_t n_db, int k) {
    if (!c) return TQ_EINVAL;
    if (!valid_codec(c)) return TQ_EUNSUPPORTED;
    if ((c->d != 128 && c->d != 256) || c->norm_blocks != 1) return TQ_EUNSUPPORTED;
    if (k < 1 || k > 64) return TQ_EUNSUPPORTED;
    if (n_q <= 0 || n_db < 0 || n_q > 65535 * 32) return TQ_EINVAL;  // 32 queries per block row of the grid
    if (n_db > ((int64_t)1 << 31) - 1) return TQ_EUNSUPPORTED;
    return TQ_OK;
}

size_t tq_search_workspace_bytes(const tq_codec* c, int n_q, int64_t n_db, int k) {
    if (search_check(c, n_q, n_db, k) != TQ_OK) return 0;
    int nb;
    int64_t rows;
    tqi::search_plan(n_q, n_db, k, c->d, c->bits, &nb, &rows);
    return tqi::search_workspace(n_q, c->d, c->qjl_m, k, nb);
}

size_t tq_workspace_bytes(int op, const tq_codec* kc, const tq_codec* vc, int batch, int n_q_heads, int n_kv_heads,
                          int64_t ctx_cap, int n_q, int64_t n_db, int k) {
    switch (op) {
        case TQ_OP_ATTN_DECODE:
        case TQ_OP_ATTN_DECODE_RW: return tq_attn_workspace_bytes(kc, vc, batch, n_q_heads, n_kv_heads, ctx_cap);
        case TQ_OP_IP_SEARCH: return tq_search_workspace_bytes(kc, n_q, n_db, k);
        case TQ_OP_ATTN_DECODE_MQ: return attn_ws_bytes(kc, vc, batch, n_q, n_q_heads, n_kv_heads, ctx_cap);
        default: return 0;
    }
}

int tq_ip_search(const tq_codec* c, const float* q, int n_q, const uint8_t* codes, const uint16_t* norms,
                 const uint8_t* qjl_bits, const uint16_t* qjl_gamma, const float* qjl_S, int64_t n_db, int k,
                 float* out_scores, int64_t* out_ids, void* workspace, size_t workspace_bytes, void* stream) {
    const int rc = search_check(c, n_q, n_db, k);
    if (rc != TQ_OK) return rc;
    if (!q || !out_scores || !out_ids || !aligned(q, 16)) return TQ_EINVAL;
    if (n_db > 0 && (!codes || !norms || !aligned(codes, 16) || !aligned(norms, 2))) return TQ_EINVAL;
    if (c->qjl_m > 0 && n_db > 0 && (!qjl_bits || !qjl_gamma || !aligned(qjl_bits, 4))) return TQ_EINVAL;
    if (needs_S(c) && !qjl_S) return TQ_EINVAL;
    int nb;
    int64_t rows;
    tqi::search_plan(n_q, n_db, k, c->d, c->bits, &nb, &rows);
    const size_t need = tqi::search_workspace(n_q, c->d, c->qjl_m, k, nb);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return TQ_EWORKSPACE;
    tqi::SearchArgs a;
    tqi::fill_codec_args(c, &a.c);
    a.q = q;
    a.n_q = n_q;
    a.codes = codes;
    a.norms = norms;
    a.qjl = qjl_bits;
    a.gamma = qjl_gamma;
    a.S = qjl_S;
    a.n_db = n_db;
    a.k = k;
    a.out_scores = out_scores;
    a.out_ids = out_ids;
    float* ws = (float*)workspace;
    const size_t qa = ((size_t)n_q * (c->d + c->qjl_m) + 63) & ~(size_t)63;
    const size_t cand = (((size_t)n_q * nb * k) + 63) & ~(size_t)63;
    a.qrot = ws;
    a.qproj = nullptr;
    a.cand_s = ws + qa;
    a.cand_i = (int32_t*)(ws + qa + cand);
    a.n_blocks = nb;
    a.block_rows = rows;
    return finish(tqi::launch_search(a, (hipStream_t)stream));
}

}  // extern "C"
