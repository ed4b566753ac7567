// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tqi {

// Everything one encode/decode launch needs, passed by value as a kernel argument.
struct CodecArgs {
    uint32_t sign_mask[16];  // D for dims 0..511 (words 8.. only at d = 512)
    float centroid[16];
    float threshold[15];
    int32_t d, bits, qjl_m;
    int32_t residual;        // TQ_RES_*
    uint32_t sign_mask2[8];  // second sign basis (TQ_RES_SRHT)
    int32_t rotation;        // TQ_ROT_*
    int32_t norm_blocks;     // 1 or 2
    uint32_t sign_mask3[8];  // D3 of TQ_ROT_DOUBLE
    // the encoder's bin table (see plan_qtab): bin b = floor(z * qt_scale +
    // qt_off) of z = w / n holds at most one threshold; qt_n bins, 0 = none
    float qt_scale, qt_off, qt_inv_scale;
    int32_t qt_n;
};

// Bins of the encoder's quantizer table at most (8 bytes each in LDS).
constexpr int kQTabMax = 512;

struct EncodeArgs {
    CodecArgs c;
    const void* x;
    int64_t n;
    int64_t x_stride;  // elements
    uint8_t* codes;
    int64_t code_stride;  // bytes
    uint16_t* norms;
    const float* S;  // [m][d] or null
    uint8_t* qjl;    // [n][m/8]
    uint16_t* gamma;
    // decode-step append: with pos set, input row r = b * seq_heads + h goes to
    // output row r * cap + pos[b], and nothing is stored when pos[b] is outside
    // [0, cap)
    const int32_t* pos;
    int64_t cap;
    int seq_heads;
    // chunked prefill (pos unset, grp_rows > 0): input row r goes to output row
    // (r / grp_rows) * cap + grp_off + r % grp_rows
    int64_t grp_rows;
    int64_t grp_off;
};

struct DecodeArgs {
    CodecArgs c;
    const uint8_t* codes;
    int64_t code_stride;
    const uint16_t* norms;
    int64_t n;
    float* out;
};

// Decode-attention launch description (see tq_attn.hip).
struct AttnArgs {
    CodecArgs kc, vc;
    const void* q;
    int q_dtype;
    int batch, hq, hkv, g;   // g = hq / hkv
    int ncols;               // query columns per sequence (1: single-token decode)
    int heads_per_chunk;     // G: query rows (of the g * ncols of a kv head) per block
    int chunks;              // g * ncols / G
    const int32_t* ctx_len;
    int64_t ctx_cap;
    const uint8_t* k_codes;
    const uint16_t* k_norms;
    const uint8_t* k_qjl;
    const uint16_t* k_gamma;
    const float* S;
    const uint8_t* v_codes;
    const uint16_t* v_norms;
    float scale;
    // score factor alpha(N) of a row attending over N tokens: mode 0 plain,
    // 1 sharpen 1 + sharp_c sqrt(ln N), 2 soften sqnr / (sqnr + sqrt(ln N * inv_ln_n0))
    int score_mode;
    float sharp_c, sqnr, inv_ln_n0;
    // sparse V: softmax weights below 2^sparse_log2 (relative to the reference
    // max) add nothing to the V sums; -INFINITY when off
    float sparse_log2;
    float* out;
    float* qproj;     // [batch][hq][m]  scale*log2e*sqrt(pi/2)/m * S H(D_K q)/sqrt(d)
    float* part;      // [batch][hq][splits][d + 2]
    int splits;
    int64_t split_tokens;  // tokens per split (multiple of 64)
    // residual window of exact tokens: [batch][hkv][win_cap][d] in win_dtype
    const void* k_win;
    const void* v_win;
    int win_dtype;
    const int32_t* win_len;  // [batch]
    int win_cap;             // 0: no window
};

// Host-side helpers.
void fill_codec_args(const tq_codec* c, CodecArgs* a);

// Launchers (return hipError_t of the launch).
hipError_t launch_encode(const EncodeArgs& a, int dtype, hipStream_t s);
// a layer's K and V encodes (same d and dtype) in one launch when neither uses QJL
hipError_t launch_encode_pair(const EncodeArgs& k, const EncodeArgs& v, int dtype, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
enum AttnStage { ATTN_PREPARE = 1, ATTN_SCAN = 2, ATTN_COMBINE = 4, ATTN_ALL = 7, ATTN_WINDOW = 8 };
hipError_t launch_attn(const AttnArgs& a, int stages, hipStream_t s);
void attn_plan(int batch, int hkv, int gv, int64_t ctx_cap, int d, int kb, int vb, bool qjl, int* splits,
               int64_t* split_tokens, int* heads_per_chunk);
// Head dimension 512: the wide kernel (tq_attn_wide_mc.hip, the dims split
// across a block's waves) in place of the scan, with its own plan.
bool attn_wide(int d);
void wide_plan(int batch, int hkv, int g, int64_t ctx_cap, int* splits, int64_t* split_tokens, int* heads_per_chunk);
hipError_t launch_wide(const AttnArgs& a, hipStream_t s);
template <int D, int KB>
hipError_t launch_split_dk(const AttnArgs& a, hipStream_t s);
template <int D, int KB>
int split_blocks_dk(int vb, bool qjl);
size_t attn_workspace(int batch, int hq, int d, int m, int splits);
// Compute units of the current device (cached per device; 1 without one).
int device_cus();

struct SearchArgs {
    CodecArgs c;
    const float* q;
    int n_q;
    const uint8_t* codes;
    const uint16_t* norms;
    const uint8_t* qjl;
    const uint16_t* gamma;
    const float* S;
    int64_t n_db;
    int k;
    float* out_scores;
    int64_t* out_ids;
    float* qrot;   // [n_q][d]
    float* qproj;  // [n_q][m]
    float* cand_s;  // [n_q][n_blocks][k]
    int32_t* cand_i;
    int n_blocks;
    int64_t block_rows;
};
hipError_t launch_search(const SearchArgs& a, hipStream_t s);
void search_plan(int n_q, int64_t n_db, int k, int d, int bits, int* n_blocks, int64_t* block_rows);
size_t search_workspace(int n_q, int d, int m, int k, int n_blocks);

}  // namespace tqi
