// EXTEND (bf16 and FP8 pools): the support check and the dispatch on the group size G. The
// kernel is in extend_attn_kernel.h; each power-of-two group size is compiled in its own
// translation unit (extend_g1.hip .. extend_g32.hip), every other one in extend_g0.hip.
#include "rax_launch.h"

namespace rax {

// Any group size whose query heads fit the 256-row tile at least once: powers of two up to 32
// have their own instantiation, every other one (3, 5, 6, 7, 12, 64, ...) the run-time one.
bool extend_bf16_supported(int32_t group, int32_t head_dim) {
    return (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 256;
}

int launch_extend_bf16(const AttnArgs& a, hipStream_t stream) {
    switch (a.n_q_heads / a.n_kv_heads) {
        case 1: return launch_extend_g1(a, stream);
        case 2: return launch_extend_g2(a, stream);
        case 4: return launch_extend_g4(a, stream);
        case 8: return launch_extend_g8(a, stream);
        case 16: return launch_extend_g16(a, stream);
        case 32: return launch_extend_g32(a, stream);
        default: return launch_extend_g0(a, stream);
    }
}

}  // namespace rax
