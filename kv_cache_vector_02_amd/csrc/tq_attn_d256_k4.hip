// Split-K decode attention kernels for d=256, 4-bit keys (all value widths
// and switch variants).  One translation unit per (d, key bits) keeps the
// template instantiations compiling in parallel.
#include "tq_attn_kernels.h"

namespace tqi {
template <>
hipError_t launch_split_dk<256, 4>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<256, 4>(a, s);
}
template <>
int split_blocks_dk<256, 4>(int vb, bool qjl) {
    return attn::split_blocks_dk<256, 4>(vb, qjl);
}
}  // namespace tqi
