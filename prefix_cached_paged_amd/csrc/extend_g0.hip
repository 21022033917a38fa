// EXTEND kernels for every group size without its own instantiation (3, 5, 6, 7, 12, 64, ...; up
// to 256 query heads per kv head): the group size is read at run time (head_dim 64 and 128, bf16
// and FP8 pools).
#include "extend_attn_kernel.h"

namespace rax {

int launch_extend_g0(const AttnArgs& a, hipStream_t stream) { return launch_extend_group<0>(a, stream); }

}  // namespace rax
