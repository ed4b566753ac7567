// Split-K decode attention kernels for d=128, 4-bit keys (all value widths
// and head-chunk sizes).  One translation unit per (d, key bits) keeps the
// template instantiations compiling in parallel.
#include "tq_attn_kernels.h"

namespace tqi {
template <>
hipError_t launch_split_dk<128, 4>(const AttnArgs& a, hipStream_t s) {
    return attn::launch_split_dk<128, 4>(a, s);
}
}  // namespace tqi
