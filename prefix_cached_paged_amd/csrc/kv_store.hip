// kv_store: scatter new K/V rows into pool slots by index.
//
// The attention layer writes its freshly computed K and V at the batch's output slot locations
// before reading the pool ("Origins: the paper and the first commit", section "Execution:
// RadixAttention and two sets of kernels"). A pool row (all kv heads of one slot) is
// n_kv_heads * head_dim contiguous elements, so each row is one contiguous copy.
//
// Work split: one 16-byte vector per thread; consecutive threads cover consecutive vectors of
// a row, so both the read of the new rows and the write of the pool row are fully coalesced.
// The copy is bitwise (no arithmetic), so one kernel serves every element format.
#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

__global__ __launch_bounds__(256) void kv_store_kernel(const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        const int32_t* __restrict__ loc,
                                                        int64_t total_vecs, int32_t row_vecs,
                                                        uint4* __restrict__ k_pool,
                                                        uint4* __restrict__ v_pool) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_vecs; i += stride) {
        const int64_t row = i / row_vecs;
        const int32_t col = (int32_t)(i - row * row_vecs);
        const int64_t dst = (int64_t)loc[row] * row_vecs + col;
        k_pool[dst] = k_new[i];
        v_pool[dst] = v_new[i];
    }
}

int launch_kv_store(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                    void* k_pool, void* v_pool, int64_t row_bytes, hipStream_t stream) {
    const int32_t row_vecs = (int32_t)(row_bytes / 16);
    const int64_t total = n_new * row_vecs;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)k_new, (const uint4*)v_new, loc, total, row_vecs,
                       (uint4*)k_pool, (uint4*)v_pool);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace rax
