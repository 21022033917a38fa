// C ABI of librax: host-side argument checks, then kernel launches on the caller's stream.
// Semantics, layouts, ownership and error behaviour of each call are documented in librax.h.
#include "librax.h"
#include "rax_launch.h"
#include "rax_check.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int32_t kMaxGridYZ = 65535;

bool dtype_ok(int dt) { return dt == RAX_BF16 || dt == RAX_FP32; }
bool scale_ok(float s) { return s == s && s > 0.f && s <= 3.4028234663852886e38f; }
size_t elem_bytes(int dt) { return dt == RAX_BF16 ? 2 : 4; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
// log2 of a page size (a power of two from 1 to 2^20), -1 otherwise.
int page_shift_of(int32_t page_size) {
    if (page_size < 1 || page_size > (1 << 20) || (page_size & (page_size - 1))) return -1;
    int s = 0;
    while ((1 << s) < page_size) ++s;
    return s;
}

rax_status check_heads(int32_t hq, int32_t hkv, int32_t d) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || hq > kMaxGridYZ) return RAX_ERR_SHAPE;
    if (!head_dim_ok(d)) return RAX_ERR_UNSUPPORTED;
    return RAX_OK;
}

}  // namespace

extern "C" {

int rax_version(void) { return kVersion; }

const char* rax_status_str(rax_status status) {
    switch (status) {
        case RAX_OK: return "RAX_OK";
        case RAX_ERR_NULL: return "RAX_ERR_NULL";
        case RAX_ERR_SHAPE: return "RAX_ERR_SHAPE";
        case RAX_ERR_DTYPE: return "RAX_ERR_DTYPE";
        case RAX_ERR_UNSUPPORTED: return "RAX_ERR_UNSUPPORTED";
        case RAX_ERR_WORKSPACE: return "RAX_ERR_WORKSPACE";
        case RAX_ERR_LAUNCH: return "RAX_ERR_LAUNCH";
        case RAX_ERR_SCRATCH: return "RAX_ERR_SCRATCH";
        default: return "unknown status";
    }
}

rax_status rax_kv_store(rax_dtype dtype, const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                        void* k_pool, void* v_pool, int64_t num_slots, int32_t n_kv_heads, int32_t head_dim,
                        hipStream_t stream) {
    if (!dtype_ok(dtype)) return RAX_ERR_DTYPE;
    if (n_new < 0 || num_slots <= 0 || n_kv_heads <= 0 || n_new > num_slots) return RAX_ERR_SHAPE;
    if (!head_dim_ok(head_dim)) return RAX_ERR_UNSUPPORTED;
    if (n_new == 0) return RAX_OK;
    if (!k_new || !v_new || !loc || !k_pool || !v_pool) return RAX_ERR_NULL;
    const int64_t row_bytes = (int64_t)n_kv_heads * head_dim * (int64_t)elem_bytes(dtype);
    if (n_new * (row_bytes / 16) > ((int64_t)1 << 62)) return RAX_ERR_SHAPE;
    return rax::launch_kv_store(k_new, v_new, loc, n_new, k_pool, v_pool, row_bytes,
                                (hipStream_t)stream) == 0 ? RAX_OK : RAX_ERR_LAUNCH;
}

size_t rax_extend_workspace_bytes(rax_dtype dtype, int32_t batch, int64_t total_extend_tokens,
                                  int32_t max_extend_len, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim) {
    // the partials of the key splits over bf16 or FP8 pools (0 when unsplit); the fp32 path
    // uses none.
    if ((dtype != RAX_BF16 && dtype != RAX_FP8_E4M3) || batch <= 0 || total_extend_tokens <= 0 || max_extend_len <= 0 ||
        n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 ||
        !rax::extend_bf16_supported(n_q_heads / n_kv_heads, head_dim))
        return 0;
    const int32_t S = rax::extend_splits(batch, n_q_heads, n_kv_heads, max_extend_len, max_seq_len);
    return rax::extend_split_workspace(S, total_extend_tokens, n_q_heads, head_dim);
}

size_t rax_decode_workspace_bytes(rax_dtype dtype, int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim) {
    if ((dtype != RAX_BF16 && dtype != RAX_FP8_E4M3) || batch <= 0 || max_seq_len <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 ||
        head_dim <= 0)
        return 0;
    return rax::decode_workspace(batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                                 dtype == RAX_FP8_E4M3);
}

int32_t rax_decode_num_splits(rax_dtype dtype, int32_t batch, int32_t max_seq_len, int32_t n_kv_heads) {
    if (dtype != RAX_BF16 && dtype != RAX_FP8_E4M3) return 1;
    if (batch <= 0 || max_seq_len <= 0 || n_kv_heads <= 0) return 1;
    return rax::decode_grid(batch, max_seq_len, n_kv_heads, dtype == RAX_FP8_E4M3);
}

}  // extern "C"

namespace {

// Checks and launch shared by the bf16/fp32 and FP8-pool EXTEND entry points.
rax_status extend_call(int dtype, bool kv8, const void* q, void* o, const void* k_pool, const void* v_pool,
                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                const int32_t* req_pool_indices, const int32_t* prefix_lens,
                const int32_t* extend_lens, const int32_t* extend_start_loc, int32_t batch,
                int64_t total_extend_tokens, int32_t max_extend_len, int32_t max_seq_len,
                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                hipStream_t stream, bool ragged = false, const void* k_new = nullptr,
                const void* v_new = nullptr, const int32_t* store_loc = nullptr,
                int32_t page_shift = 0) {
    if (!dtype_ok(dtype)) return RAX_ERR_DTYPE;
    if (batch < 0 || batch > kMaxGridYZ || total_extend_tokens < 0 || max_extend_len < 0 ||
        max_seq_len < 0 || num_slots <= 0 || r2t_stride <= 0 ||
        max_seq_len > (r2t_stride << page_shift) || max_extend_len > max_seq_len ||
        max_extend_len > total_extend_tokens)
        return RAX_ERR_SHAPE;
    const rax_status st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != RAX_OK) return st;
    const int32_t G = n_q_heads / n_kv_heads;
    if (dtype == RAX_BF16 && !rax::extend_bf16_supported(G, head_dim)) return RAX_ERR_UNSUPPORTED;
    if (!(sm_scale == sm_scale)) return RAX_ERR_SHAPE;
    if (kv8 && (!scale_ok(k_scale) || !scale_ok(v_scale))) return RAX_ERR_SHAPE;
    if (batch == 0 || total_extend_tokens == 0 || max_extend_len == 0) return RAX_OK;
    if (!q || !o || !k_pool || !v_pool || !req_to_token || !req_pool_indices || !prefix_lens ||
        !extend_lens || !extend_start_loc)
        return RAX_ERR_NULL;
    if (ragged && (!k_new || !v_new)) return RAX_ERR_NULL;
    const size_t need = rax_extend_workspace_bytes(kv8 ? RAX_FP8_E4M3 : (rax_dtype)dtype, batch,
                                                   total_extend_tokens, max_extend_len, max_seq_len,
                                                   n_q_heads, n_kv_heads, head_dim);
    if (need > 0 && (!workspace || workspace_bytes < need)) return RAX_ERR_WORKSPACE;

    rax::AttnArgs a{};
    a.q = q; a.o = o; a.k_pool = k_pool; a.v_pool = v_pool; a.num_slots = num_slots;
    a.r2t = req_to_token; a.r2t_stride = r2t_stride; a.req_pool_indices = req_pool_indices;
    a.prefix_lens = prefix_lens; a.extend_lens = extend_lens; a.extend_start_loc = extend_start_loc;
    a.total_tokens = total_extend_tokens; a.max_extend_len = max_extend_len;
    a.seq_lens = nullptr; a.batch = batch; a.max_seq_len = max_seq_len;
    a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads; a.head_dim = head_dim; a.sm_scale = sm_scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.kv8 = kv8; a.k_scale = k_scale; a.v_scale = v_scale;
    a.ragged = ragged; a.k_new = k_new; a.v_new = v_new; a.store_loc = store_loc;
    a.page_shift = page_shift;
    const int rc = dtype == RAX_BF16 ? rax::launch_extend_bf16(a, (hipStream_t)stream)
                                     : rax::launch_extend_fp32(a, (hipStream_t)stream);
    return rc == 0 ? RAX_OK : RAX_ERR_LAUNCH;
}

// Checks and launch shared by the bf16/fp32 and FP8-pool DECODE entry points.
rax_status decode_call(int dtype, bool kv8, const void* q, void* o, const void* k_pool, const void* v_pool,
                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                float sm_scale, float k_scale, float v_scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream, int32_t page_shift = 0,
                bool static_scratch = false) {
    if (!dtype_ok(dtype)) return RAX_ERR_DTYPE;
    if (batch < 0 || batch > kMaxGridYZ || max_seq_len < 0 || num_slots <= 0 || r2t_stride <= 0 ||
        max_seq_len > (r2t_stride << page_shift))
        return RAX_ERR_SHAPE;
    const rax_status st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != RAX_OK) return st;
    const int32_t G = n_q_heads / n_kv_heads;
    if (dtype == RAX_BF16 && !rax::decode_bf16_supported(G, head_dim)) return RAX_ERR_UNSUPPORTED;
    if (!(sm_scale == sm_scale)) return RAX_ERR_SHAPE;
    if (kv8 && (!scale_ok(k_scale) || !scale_ok(v_scale))) return RAX_ERR_SHAPE;
    if (batch == 0) return RAX_OK;
    if (max_seq_len == 0) return RAX_ERR_SHAPE;
    if (dtype == RAX_BF16 &&
        rax::decode_grid(batch, max_seq_len, rax::decode_wave_heads(n_q_heads, n_kv_heads), kv8) < 0)
        return RAX_ERR_SHAPE;
    if (!q || !o || !k_pool || !v_pool || !req_to_token || !req_pool_indices || !seq_lens)
        return RAX_ERR_NULL;
    const size_t need = rax_decode_workspace_bytes(kv8 ? RAX_FP8_E4M3 : (rax_dtype)dtype, batch, max_seq_len,
                                                   n_q_heads, n_kv_heads, head_dim);
    if (static_scratch && need > 0) {
        // the library's static scratch takes the place of the workspace
        if (need > RAX_DECODE_SCRATCH_BYTES) return RAX_ERR_SCRATCH;
        workspace = rax::decode_scratch(stream);
        if (workspace == nullptr) return RAX_ERR_LAUNCH;
        workspace_bytes = RAX_DECODE_SCRATCH_BYTES;
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return RAX_ERR_WORKSPACE;

    rax::AttnArgs a{};
    a.q = q; a.o = o; a.k_pool = k_pool; a.v_pool = v_pool; a.num_slots = num_slots;
    a.r2t = req_to_token; a.r2t_stride = r2t_stride; a.req_pool_indices = req_pool_indices;
    a.prefix_lens = nullptr; a.extend_lens = nullptr; a.extend_start_loc = nullptr;
    a.total_tokens = batch; a.max_extend_len = 0; a.seq_lens = seq_lens; a.batch = batch;
    a.max_seq_len = max_seq_len; a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads;
    a.head_dim = head_dim; a.sm_scale = sm_scale; a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    a.kv8 = kv8; a.k_scale = k_scale; a.v_scale = v_scale;
    a.page_shift = page_shift;
    const int rc = dtype == RAX_BF16 ? rax::launch_decode_bf16(a, (hipStream_t)stream)
                                     : rax::launch_decode_fp32(a, (hipStream_t)stream);
    return rc == 0 ? RAX_OK : RAX_ERR_LAUNCH;
}

}  // namespace

extern "C" {

rax_status rax_decode_attention(rax_dtype dtype, const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                float sm_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_call(dtype, false, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                       sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream);
}

rax_status rax_decode_attention_noalloc(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                        const void* v_pool, int64_t num_slots,
                                        const int32_t* req_to_token, int64_t r2t_stride,
                                        const int32_t* req_pool_indices, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                        hipStream_t stream) {
    return decode_call(dtype, false, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                       sm_scale, 1.f, 1.f, nullptr, 0, stream, 0, true);
}

rax_status rax_kv_store_fp8(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                            void* k_pool, void* v_pool, int64_t num_slots, int32_t n_kv_heads,
                            int32_t head_dim, float k_scale, float v_scale, hipStream_t stream) {
    if (n_new < 0 || num_slots <= 0 || n_kv_heads <= 0 || n_new > num_slots) return RAX_ERR_SHAPE;
    if (!head_dim_ok(head_dim)) return RAX_ERR_UNSUPPORTED;
    if (!scale_ok(k_scale) || !scale_ok(v_scale)) return RAX_ERR_SHAPE;
    if (n_new == 0) return RAX_OK;
    if (!k_new || !v_new || !loc || !k_pool || !v_pool) return RAX_ERR_NULL;
    const int64_t row_elems = (int64_t)n_kv_heads * head_dim;
    if (n_new * (row_elems / 8) > ((int64_t)1 << 62)) return RAX_ERR_SHAPE;
    const float k_inv = (float)(1.0 / (double)k_scale);
    const float v_inv = (float)(1.0 / (double)v_scale);
    return rax::launch_kv_store_fp8(k_new, v_new, loc, n_new, k_pool, v_pool, row_elems, k_inv, v_inv,
                                    (hipStream_t)stream) == 0 ? RAX_OK : RAX_ERR_LAUNCH;
}

rax_status rax_decode_attention_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                    int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                    const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                                    int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_call(RAX_BF16, true, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                       sm_scale, k_scale, v_scale, workspace, workspace_bytes, stream);
}

rax_status rax_extend_attention(rax_dtype dtype, const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                const int32_t* extend_lens, const int32_t* extend_start_loc, int32_t batch,
                                int64_t total_extend_tokens, int32_t max_extend_len, int32_t max_seq_len,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return extend_call(dtype, false, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream);
}

rax_status rax_extend_attention_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                    int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                    const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                    const int32_t* extend_lens, const int32_t* extend_start_loc,
                                    int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                    int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return extend_call(RAX_BF16, true, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, k_scale, v_scale, workspace, workspace_bytes, stream);
}

rax_status rax_extend_attention_ragged(rax_dtype dtype, const void* q, void* o, const void* k_new,
                                       const void* v_new, const int32_t* store_loc, void* k_pool,
                                       void* v_pool, int64_t num_slots, const int32_t* req_to_token,
                                       int64_t r2t_stride, const int32_t* req_pool_indices,
                                       const int32_t* prefix_lens, const int32_t* extend_lens,
                                       const int32_t* extend_start_loc, int32_t batch,
                                       int64_t total_extend_tokens, int32_t max_extend_len,
                                       int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, float sm_scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (total_extend_tokens > 0 && store_loc && total_extend_tokens > num_slots) return RAX_ERR_SHAPE;
    return extend_call(dtype, false, q, o, k_pool, v_pool, num_slots, req_to_token, r2t_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream, true, k_new,
                       v_new, store_loc);
}

rax_status rax_extend_attention_paged(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                      const void* v_pool, int64_t num_slots, const int32_t* page_table,
                                      int64_t pt_stride, int32_t page_size,
                                      const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                      const int32_t* extend_lens, const int32_t* extend_start_loc,
                                      int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                      int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, float sm_scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || (pt_stride > 0 && pt_stride > (INT64_MAX >> 21))) return RAX_ERR_SHAPE;
    return extend_call(dtype, false, q, o, k_pool, v_pool, num_slots, page_table, pt_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream, false,
                       nullptr, nullptr, nullptr, ps);
}

rax_status rax_decode_attention_paged(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                      const void* v_pool, int64_t num_slots, const int32_t* page_table,
                                      int64_t pt_stride, int32_t page_size,
                                      const int32_t* req_pool_indices, const int32_t* seq_lens,
                                      int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || (pt_stride > 0 && pt_stride > (INT64_MAX >> 21))) return RAX_ERR_SHAPE;
    return decode_call(dtype, false, q, o, k_pool, v_pool, num_slots, page_table, pt_stride,
                       req_pool_indices, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                       sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream, ps);
}

rax_status rax_extend_attention_ragged_paged(rax_dtype dtype, const void* q, void* o, const void* k_new,
                                             const void* v_new, const int32_t* store_loc, void* k_pool,
                                             void* v_pool, int64_t num_slots, const int32_t* page_table,
                                             int64_t pt_stride, int32_t page_size,
                                             const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                             const int32_t* extend_lens, const int32_t* extend_start_loc,
                                             int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                             int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, float sm_scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || (pt_stride > 0 && pt_stride > (INT64_MAX >> 21))) return RAX_ERR_SHAPE;
    if (total_extend_tokens > 0 && store_loc && total_extend_tokens > num_slots) return RAX_ERR_SHAPE;
    return extend_call(dtype, false, q, o, k_pool, v_pool, num_slots, page_table, pt_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, 1.f, 1.f, workspace, workspace_bytes, stream, true, k_new,
                       v_new, store_loc, ps);
}

rax_status rax_extend_attention_paged_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                          int64_t num_slots, const int32_t* page_table, int64_t pt_stride,
                                          int32_t page_size, const int32_t* req_pool_indices,
                                          const int32_t* prefix_lens, const int32_t* extend_lens,
                                          const int32_t* extend_start_loc, int32_t batch,
                                          int64_t total_extend_tokens, int32_t max_extend_len,
                                          int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || (pt_stride > 0 && pt_stride > (INT64_MAX >> 21))) return RAX_ERR_SHAPE;
    return extend_call(RAX_BF16, true, q, o, k_pool, v_pool, num_slots, page_table, pt_stride,
                       req_pool_indices, prefix_lens, extend_lens, extend_start_loc, batch,
                       total_extend_tokens, max_extend_len, max_seq_len, n_q_heads, n_kv_heads,
                       head_dim, sm_scale, k_scale, v_scale, workspace, workspace_bytes, stream, false,
                       nullptr, nullptr, nullptr, ps);
}

rax_status rax_decode_attention_paged_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                          int64_t num_slots, const int32_t* page_table, int64_t pt_stride,
                                          int32_t page_size, const int32_t* req_pool_indices,
                                          const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                          float sm_scale, float k_scale, float v_scale, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || (pt_stride > 0 && pt_stride > (INT64_MAX >> 21))) return RAX_ERR_SHAPE;
    return decode_call(RAX_BF16, true, q, o, k_pool, v_pool, num_slots, page_table, pt_stride,
                       req_pool_indices, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim,
                       sm_scale, k_scale, v_scale, workspace, workspace_bytes, stream, ps);
}

}  // extern "C"

static_assert(RAX_CHECK_LENGTH == rax::kCheckLength && RAX_CHECK_ROW == rax::kCheckRow &&
                  RAX_CHECK_SLOT == rax::kCheckSlot && RAX_CHECK_DUPLICATE == rax::kCheckDuplicate &&
                  RAX_CHECK_OVERLAP == rax::kCheckOverlap && RAX_CHECK_COUNT == rax::kCheckCount,
              "rax_check_item and the kernels' counters must agree");

namespace {

// Host checks and launch shared by rax_check_extend and rax_check_decode.
rax_status check_requests(bool ext, const int32_t* table, int64_t table_rows, int64_t table_stride,
                   int32_t page_size, const int32_t* rpi, const int32_t* lens_a,
                   const int32_t* lens_b, const int32_t* start, int32_t batch, int64_t total,
                   int32_t max_ext, int32_t max_seq, int64_t num_slots, bool ragged,
                   const int32_t* store_loc, void* workspace, size_t workspace_bytes,
                   int32_t* counts, hipStream_t stream) {
    const int ps = page_shift_of(page_size);
    if (ps < 0 || batch < 0 || table_stride <= 0 || table_stride > (INT64_MAX >> 21) ||
        max_seq < 0 || max_seq > (table_stride << ps) || num_slots <= 0 || total < 0 ||
        max_ext < 0 || (batch > 0 && table_rows <= 0) || (store_loc && !ragged))
        return RAX_ERR_SHAPE;
    if (!counts) return RAX_ERR_NULL;
    if (batch > 0 && (!table || !rpi || !lens_a || (ext && (!lens_b || !start)))) return RAX_ERR_NULL;
    const bool marks = store_loc != nullptr && total > 0;
    if (marks && (!workspace || workspace_bytes < rax_check_workspace_bytes(num_slots)))
        return RAX_ERR_WORKSPACE;
    rax::CheckArgs c{};
    c.table = table; c.table_rows = table_rows; c.stride = table_stride; c.page_shift = ps;
    c.rpi = rpi; c.lens_a = lens_a; c.lens_b = ext ? lens_b : nullptr; c.start = ext ? start : nullptr;
    c.total = total; c.max_ext = max_ext; c.max_seq = max_seq; c.num_slots = num_slots;
    c.ragged = ragged; c.store_loc = marks ? store_loc : nullptr; c.bitmap = workspace;
    c.counts = counts; c.batch = batch;
    return rax::launch_check_requests(c, (hipStream_t)stream) == 0 ? RAX_OK : RAX_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t rax_check_workspace_bytes(int64_t num_slots) {
    return num_slots > 0 ? (size_t)rax::check_bitmap_words(num_slots) * sizeof(uint32_t) : 0;
}

rax_status rax_check_kv_store(const int32_t* loc, int64_t n_new, int64_t num_slots, void* workspace,
                              size_t workspace_bytes, int32_t* counts, hipStream_t stream) {
    if (n_new < 0 || num_slots <= 0) return RAX_ERR_SHAPE;
    if (!counts || (n_new > 0 && !loc)) return RAX_ERR_NULL;
    if (!workspace || workspace_bytes < rax_check_workspace_bytes(num_slots)) return RAX_ERR_WORKSPACE;
    return rax::launch_check_store(loc, n_new, num_slots, workspace, counts, (hipStream_t)stream) == 0
               ? RAX_OK
               : RAX_ERR_LAUNCH;
}

rax_status rax_check_extend(const int32_t* table, int64_t table_rows, int64_t table_stride,
                            int32_t page_size, const int32_t* req_pool_indices, const int32_t* prefix_lens,
                            const int32_t* extend_lens, const int32_t* extend_start_loc, int32_t batch,
                            int64_t total_extend_tokens, int32_t max_extend_len, int32_t max_seq_len,
                            int64_t num_slots, int32_t ragged, const int32_t* store_loc, void* workspace,
                            size_t workspace_bytes, int32_t* counts, hipStream_t stream) {
    return check_requests(true, table, table_rows, table_stride, page_size, req_pool_indices,
                          prefix_lens, extend_lens, extend_start_loc, batch, total_extend_tokens,
                          max_extend_len, max_seq_len, num_slots, ragged != 0, store_loc, workspace,
                          workspace_bytes, counts, stream);
}

rax_status rax_check_decode(const int32_t* table, int64_t table_rows, int64_t table_stride,
                            int32_t page_size, const int32_t* req_pool_indices, const int32_t* seq_lens,
                            int32_t batch, int32_t max_seq_len, int64_t num_slots, int32_t* counts,
                            hipStream_t stream) {
    return check_requests(false, table, table_rows, table_stride, page_size, req_pool_indices,
                          seq_lens, nullptr, nullptr, batch, 0, 0, max_seq_len, num_slots, false,
                          nullptr, nullptr, 0, counts, stream);
}

}  // extern "C"
