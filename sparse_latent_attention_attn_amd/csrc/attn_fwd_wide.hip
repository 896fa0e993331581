// The wide bf16 key loop (d = 512, 4 waves of two 16-head blocks each). It sits in a
// translation unit of its own because it is compiled with the MFMA accumulators in AGPRs:
// its O (256 accumulators per lane) cannot live in VGPRs, while the other shapes run best
// with VGPR accumulators (see build_lib.py).
#include "attn_fwd_kernel.hpp"

namespace sa {

hipError_t launch_fwd_wide(const KParams& p, int blocks, hipStream_t st) {
    return launch_fwd<512, false, 4, 2>(p, blocks, st);
}

}  // namespace sa
