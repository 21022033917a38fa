// EXTEND kernels for 8 query heads per kv head (head_dim 64 and 128, bf16 and FP8 pools).
#include "extend_attn_kernel.h"

namespace rax {

int launch_extend_g8(const AttnArgs& a, hipStream_t stream) { return launch_extend_group<8>(a, stream); }

}  // namespace rax
