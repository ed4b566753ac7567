// Split-K decode attention kernels for d=128, 2-bit keys (all value widths
// and switch variants).  One translation unit per (d, key bits) keeps the
// template instantiations compiling in parallel.
#include "tq_attn_kernels.h"

namespace tqi {
template <>
hipError_t launch_split_dk<128, 2>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<128, 2>(a, s);
}
template <>
int split_blocks_dk<128, 2>(int vb, bool qjl) {
    return attn::split_blocks_dk<128, 2>(vb, qjl);
}
}  // namespace tqi
