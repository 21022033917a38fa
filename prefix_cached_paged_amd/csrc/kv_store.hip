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

// Store into FP8 E4M3 pools ("Inside SGLang", Step 6: an FP8 KV cache holds one byte per
// element, with a scale per tensor). Each bf16 element is widened to float32 (exact),
// multiplied by the float32 reciprocal of the pool's scale, clamped to +-448 (the largest
// finite E4M3 magnitude; a NaN in the pool would poison every query reading it) and rounded to
// the nearest E4M3 value, ties to even, by the hardware conversion. One thread turns one
// 8-element piece (16 bytes of bf16) into 8 bytes; accesses stay coalesced as above.
namespace {

__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float inv) {
    const float a = fminf(fmaxf(__uint_as_float(w0 << 16) * inv, -448.f), 448.f);
    const float b = fminf(fmaxf(__uint_as_float(w0 & 0xFFFF0000u) * inv, -448.f), 448.f);
    const float c = fminf(fmaxf(__uint_as_float(w1 << 16) * inv, -448.f), 448.f);
    const float d = fminf(fmaxf(__uint_as_float(w1 & 0xFFFF0000u) * inv, -448.f), 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0, 1
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);       // bytes 2, 3
    return (uint32_t)r;
}

}  // namespace

__global__ __launch_bounds__(256) void kv_store_fp8_kernel(const uint4* __restrict__ k_new,
                                                            const uint4* __restrict__ v_new,
                                                            const int32_t* __restrict__ loc,
                                                            int64_t total_units, int32_t row_units,
                                                            uint2* __restrict__ k_pool,
                                                            uint2* __restrict__ v_pool,
                                                            float k_inv, float v_inv) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_units; i += stride) {
        const int64_t row = i / row_units;
        const int32_t col = (int32_t)(i - row * row_units);
        const int64_t dst = (int64_t)loc[row] * row_units + col;
        const uint4 k = k_new[i];
        const uint4 v = v_new[i];
        k_pool[dst] = make_uint2(e4m3x4(k.x, k.y, k_inv), e4m3x4(k.z, k.w, k_inv));
        v_pool[dst] = make_uint2(e4m3x4(v.x, v.y, v_inv), e4m3x4(v.z, v.w, v_inv));
    }
}

int launch_kv_store_fp8(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                        void* k_pool, void* v_pool, int64_t row_elems, float k_inv, float v_inv,
                        hipStream_t stream) {
    const int32_t row_units = (int32_t)(row_elems / 8);
    const int64_t total = n_new * row_units;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(kv_store_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)k_new, (const uint4*)v_new, loc, total, row_units,
                       (uint2*)k_pool, (uint2*)v_pool, k_inv, v_inv);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace rax
