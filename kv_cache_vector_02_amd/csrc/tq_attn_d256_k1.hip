// Split-K decode attention kernels for d=256, 1-bit keys (all value widths
// and switch variants).  One translation unit per (d, key bits) keeps the
// template instantiations compiling in parallel.
#include "tq_attn_kernels.h"

namespace tqi {
template <>
hipError_t launch_split_dk<256, 1>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<256, 1>(a, s);
}
template <>
int split_blocks_dk<256, 1>(int vb, bool qjl) {
    return attn::split_blocks_dk<256, 1>(vb, qjl);
}
}  // namespace tqi
