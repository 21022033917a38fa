// EXTEND and DECODE attention in fp32 (vector ALU, fp32 arithmetic end to end).
//
// Same definition as the bf16 kernels ("Inside SGLang", Step 3: Q K^T, scale, causal mask,
// row softmax, times V, over keys gathered through req_to_token), for pools stored in fp32.
// No reduced-precision matrix instructions are used, so results stay within fp32 rounding.
//
// One wave per (query row, query head). Lanes take 64 keys at a time: each lane forms the full
// dot product of the query (broadcast from LDS) with its key's row, the wave updates a running
// max and sum, then the lanes switch to head_dim and accumulate p_j * V_j with p_j and the slot
// broadcast by ds_bpermute, loading the V rows of 8 keys at a time. expf is used for the
// exponentials.
//
// The scores, the running max and the exponent argument s_j - m are formed in double precision;
// everything from the weights on (p_j, the row sum, P V) is fp32. The softmax turns an absolute
// error in a score into a relative error of its weight, and an fp32 score of magnitude ~50 (a
// sharply peaked row) already carries ~2e-6 of rounding, which moves O(1) outputs by ~1e-5. The
// argument s_j - m of the keys that carry weight is small, so its single rounding to fp32 is
// harmless; downstream the errors stay relative to the weights.
#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

namespace {

// RAG (EXTEND only): key positions j >= prefix come from new row s0 + j - prefix of k_new /
// v_new ([tokens, Hkv, D]) instead of the pool.
// PG: r2t is a page table (page size 2^page_shift): position j lives at slot
// r2t[row, j >> page_shift] << page_shift | (j & (2^page_shift - 1)).
template <int D, bool CAUSAL, bool RAG, bool PG>
__global__ __launch_bounds__(64) void attn_rows_fp32_kernel(
    const float* __restrict__ q, float* __restrict__ o, const float* __restrict__ k_pool,
    const float* __restrict__ v_pool, const float* __restrict__ k_new, const float* __restrict__ v_new,
    const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ extend_start_loc,
    const int32_t* __restrict__ seq_lens, int64_t total_tokens, int32_t max_extend_len,
    int32_t max_seq_len, int32_t Hq, int32_t Hkv, float sm_scale, int32_t page_shift) {
    constexpr int PER = D / 64;
    __shared__ float qs[D];
    const int lane = threadIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int G = Hq / Hkv;
    const int g = h / G;

    int64_t qrow;
    int nkeys;
    int pre = 0, s0 = 0;  // RAG: prefix length and first row of the request's new rows
    if (CAUSAL) {
        const int i = blockIdx.x;
        int e = min(extend_lens[b], max_extend_len);
        s0 = extend_start_loc[b];
        e = (int)min((int64_t)e, total_tokens - s0);
        if (i >= e) return;
        pre = prefix_lens[b];
        nkeys = min(pre + i + 1, max_seq_len);
        qrow = (int64_t)(s0 + i);
    } else {
        nkeys = min(seq_lens[b], max_seq_len);
        qrow = b;
    }
    float* orow = o + (qrow * Hq + h) * D;
    if (nkeys <= 0) {
#pragma unroll
        for (int k = 0; k < PER; ++k) orow[64 * k + lane] = 0.f;
        return;
    }
    const float* qr = q + (qrow * Hq + h) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) qs[64 * k + lane] = qr[64 * k + lane];
    __syncthreads();

    const int32_t* row = r2t + (int64_t)rpi[b] * r2t_stride;
    const int64_t pool_row = (int64_t)Hkv * D;
    double m = -INFINITY;
    float lsum = 0.f;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;

    for (int j0 = 0; j0 < nkeys; j0 += 64) {
        const int j = j0 + lane;
        const bool ok = j < nkeys;
        const int jc = ok ? j : nkeys - 1;
        const int slot = (RAG && jc >= pre) ? 0
                         : PG ? (row[jc >> page_shift] << page_shift) | (jc & ((1 << page_shift) - 1))
                              : row[jc];
        const float* kr = (RAG && jc >= pre) ? k_new + (int64_t)(s0 + jc - pre) * pool_row + (int64_t)g * D
                                             : k_pool + (int64_t)slot * pool_row + (int64_t)g * D;
        double dot = 0.0;  // products of two fp32 values are exact in double
        for (int d = 0; d < D; d += 4) {
            const float4 kv = *(const float4*)(kr + d);
            dot = fma((double)qs[d], (double)kv.x, dot);
            dot = fma((double)qs[d + 1], (double)kv.y, dot);
            dot = fma((double)qs[d + 2], (double)kv.z, dot);
            dot = fma((double)qs[d + 3], (double)kv.w, dot);
        }
        const double x = ok ? dot * (double)sm_scale : -INFINITY;
        double mx = x;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) mx = fmax(mx, __shfl_xor(mx, s, kWave));
        const double m_new = fmax(m, mx);
        const float alpha = expf((float)(m - m_new));  // m = -inf at the first block: alpha = 0
        m = m_new;
        const float pj = ok ? expf((float)(x - m)) : 0.f;
        float ps = pj;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) ps += __shfl_xor(ps, s, kWave);
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] *= alpha;
        // P V, 8 keys at a time: their V rows are loaded together, then added in key order.
        // Keys past the last one (lanes without a key) carry p = 0 and a clamped valid row.
        const int nj = min(64, nkeys - j0);
        for (int jj = 0; jj < nj; jj += 8) {
            float pb[8], vv[8][PER];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pb[u] = __shfl(pj, jj + u, kWave);
                const int sb = __shfl(slot, jj + u, kWave);
                const int pos = min(j0 + jj + u, nkeys - 1);
                const float* vr = (RAG && pos >= pre) ? v_new + (int64_t)(s0 + pos - pre) * pool_row + (int64_t)g * D
                                                      : v_pool + (int64_t)sb * pool_row + (int64_t)g * D;
#pragma unroll
                for (int k = 0; k < PER; ++k) vv[u][k] = vr[64 * k + lane];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int k = 0; k < PER; ++k) acc[k] = fmaf(pb[u], vv[u][k], acc[k]);
        }
    }
    const float inv = 1.f / lsum;
#pragma unroll
    for (int k = 0; k < PER; ++k) orow[64 * k + lane] = acc[k] * inv;
}

template <bool CAUSAL, bool RAG, bool PG>
int launch_rows(const AttnArgs& a, hipStream_t stream) {
    const unsigned gx = CAUSAL ? (unsigned)a.max_extend_len : 1u;
    if (gx == 0 || a.batch == 0) return 0;
    dim3 grid(gx, a.n_q_heads, a.batch);
    if (a.head_dim == 128) {
        hipLaunchKernelGGL((attn_rows_fp32_kernel<128, CAUSAL, RAG, PG>), grid, dim3(64), 0, stream,
                           (const float*)a.q, (float*)a.o, (const float*)a.k_pool, (const float*)a.v_pool,
                           (const float*)a.k_new, (const float*)a.v_new, a.r2t, a.r2t_stride, a.req_pool_indices, a.prefix_lens, a.extend_lens,
                           a.extend_start_loc, a.seq_lens, a.total_tokens, a.max_extend_len,
                           a.max_seq_len, a.n_q_heads, a.n_kv_heads, a.sm_scale, a.page_shift);
    } else {
        hipLaunchKernelGGL((attn_rows_fp32_kernel<64, CAUSAL, RAG, PG>), grid, dim3(64), 0, stream,
                           (const float*)a.q, (float*)a.o, (const float*)a.k_pool, (const float*)a.v_pool,
                           (const float*)a.k_new, (const float*)a.v_new, a.r2t, a.r2t_stride, a.req_pool_indices, a.prefix_lens, a.extend_lens,
                           a.extend_start_loc, a.seq_lens, a.total_tokens, a.max_extend_len,
                           a.max_seq_len, a.n_q_heads, a.n_kv_heads, a.sm_scale, a.page_shift);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

// Ragged fp32 EXTEND with a store: the rows are stored by the copy kernel first (no slot it
// writes is read by the attention kernel, so the order only keeps the pool consistent).
int launch_extend_fp32(const AttnArgs& a, hipStream_t stream) {
    if (!a.ragged)
        return a.page_shift ? launch_rows<true, false, true>(a, stream) : launch_rows<true, false, false>(a, stream);
    if (a.store_loc != nullptr) {
        const int64_t row_bytes = (int64_t)a.n_kv_heads * a.head_dim * 4;
        if (launch_kv_store(a.k_new, a.v_new, a.store_loc, a.total_tokens, const_cast<void*>(a.k_pool),
                            const_cast<void*>(a.v_pool), row_bytes, stream) != 0)
            return -1;
    }
    return a.page_shift ? launch_rows<true, true, true>(a, stream) : launch_rows<true, true, false>(a, stream);
}
int launch_decode_fp32(const AttnArgs& a, hipStream_t stream) {
    return a.page_shift ? launch_rows<false, false, true>(a, stream) : launch_rows<false, false, false>(a, stream);
}

}  // namespace rax
