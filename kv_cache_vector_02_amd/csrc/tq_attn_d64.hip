// Split-K decode attention kernels for d=64: 2- and 4-bit keys, 2- to 4-bit
// values (a lane group covers 16 dims, so its key bytes are a whole number of
// dwords only at 2 and 4 bits).  The head_dim 64 configurations of "TurboQuant
// KV 캐시 압축 for llama.cpp" (v1.5.3: 4-bit K, or 2-bit K with the 1-bit residual,
// with 3-bit V) fall inside this set.
#include "tq_attn_kernels.h"

namespace tqi {
template <>
hipError_t launch_split_dk<64, 2>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<64, 2>(a, s);
}
template <>
int split_blocks_dk<64, 2>(int vb, bool qjl) {
    return attn::split_blocks_dk<64, 2>(vb, qjl);
}
template <>
hipError_t launch_split_dk<64, 4>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<64, 4>(a, s);
}
template <>
int split_blocks_dk<64, 4>(int vb, bool qjl) {
    return attn::split_blocks_dk<64, 4>(vb, qjl);
}
}  // namespace tqi
