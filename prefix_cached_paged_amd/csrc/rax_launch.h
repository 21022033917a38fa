// Internal (C++) launch interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rax {

// Arguments of one EXTEND or DECODE call, already validated on the host.
struct AttnArgs {
    const void* q;
    void* o;
    const void* k_pool;
    const void* v_pool;
    int64_t num_slots;
    const int32_t* r2t;
    int64_t r2t_stride;
    const int32_t* req_pool_indices;
    // EXTEND
    const int32_t* prefix_lens;
    const int32_t* extend_lens;
    const int32_t* extend_start_loc;
    int64_t total_tokens;
    int32_t max_extend_len;
    // DECODE
    const int32_t* seq_lens;
    // both
    int32_t batch;
    int32_t max_seq_len;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    float sm_scale;
    // FP8 E4M3 pools (kv8): element = scale * e4m3(byte); 1 for bf16/fp32 pools.
    bool kv8;
    float k_scale;
    float v_scale;
    // Ragged EXTEND: suffix keys come from k_new / v_new ([total_tokens, Hkv, D], rows in q's
    // order) instead of the pool; store_loc (optional) names the pool slots they are stored to.
    bool ragged;
    const void* k_new;
    const void* v_new;
    const int32_t* store_loc;
    // Page table instead of a token table (r2t then holds pages): log2 of the page size, 0 for
    // the token-granular table.
    int32_t page_shift;
    void* workspace;
    size_t workspace_bytes;
};

// True when every byte offset slot * row_bytes + (offset within the row) of the pool fits an
// unsigned 32-bit value and slot fits 24 bits, so kernels can address rows from a uniform base
// with 32-bit offsets and a 24-bit multiply.
inline bool pool_fits_32bit_offsets(int64_t num_slots, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t elem_bytes) {
    const int64_t row = (int64_t)n_kv_heads * head_dim * elem_bytes;
    return num_slots <= ((int64_t)1 << 24) && num_slots * row <= ((int64_t)1 << 32) &&
           row < ((int64_t)1 << 24);
}

int launch_kv_store(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                    void* k_pool, void* v_pool, int64_t row_bytes, hipStream_t stream);
// bf16 rows -> FP8 E4M3 pools; k_inv / v_inv are the float32 reciprocals of the scales.
int launch_kv_store_fp8(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                        void* k_pool, void* v_pool, int64_t row_elems, float k_inv, float v_inv,
                        hipStream_t stream);

// EXTEND key splits: when the (request, kv head) pairs times the row tiles of 256 query rows
// (256 / G tokens) fill at most half a round of the 256 CUs, each row tile's keys are split
// over S workgroups, S = floor(256 / work) (so the split grid still fits one round), at most
// 16 and at most one per 8 key tiles of 64 keys (so a split streams 512 keys or more).
inline int32_t extend_splits(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t max_extend_len, int32_t max_seq_len) {
    if (batch <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return 1;
    const int32_t G = n_q_heads / n_kv_heads;
    if (G < 1 || G > 256) return 1;
    const int32_t BQ = 256 / G;
    const int64_t work = (int64_t)batch * n_kv_heads * ((max_extend_len + BQ - 1) / BQ);
    if (work <= 0 || work >= 256) return 1;
    int64_t S = 256 / work;
    const int64_t by_keys = ((int64_t)max_seq_len + 63) / 64 / 8;
    if (S > by_keys) S = by_keys;
    if (S > 16) S = 16;
    return S < 1 ? 1 : (int32_t)S;
}
// Workspace of S splits: partial rows (fp32, head_dim each) and log2-sum-exps (fp32) for
// S * total_tokens * n_q_heads rows; the log2-sum-exps start 256-byte aligned.
inline size_t extend_split_o_bytes(int32_t S, int64_t total_tokens, int32_t n_q_heads, int32_t head_dim) {
    return ((size_t)S * total_tokens * n_q_heads * head_dim * 4 + 255) / 256 * 256;
}
inline size_t extend_split_workspace(int32_t S, int64_t total_tokens, int32_t n_q_heads, int32_t head_dim) {
    if (S <= 1) return 0;
    return extend_split_o_bytes(S, total_tokens, n_q_heads, head_dim) + (size_t)S * total_tokens * n_q_heads * 4;
}

// bf16, MFMA paths.
bool extend_bf16_supported(int32_t group, int32_t head_dim);
int launch_extend_bf16(const AttnArgs& a, hipStream_t stream);
// per group size G (extend_g<G>.hip)
int launch_extend_g1(const AttnArgs& a, hipStream_t stream);
int launch_extend_g2(const AttnArgs& a, hipStream_t stream);
int launch_extend_g4(const AttnArgs& a, hipStream_t stream);
int launch_extend_g8(const AttnArgs& a, hipStream_t stream);
int launch_extend_g16(const AttnArgs& a, hipStream_t stream);
int launch_extend_g32(const AttnArgs& a, hipStream_t stream);
int launch_extend_g0(const AttnArgs& a, hipStream_t stream);  // any other group size up to 256

bool decode_bf16_supported(int32_t group, int32_t head_dim);
// Waves per range of the split kernel: one per kv head, ceil(G / 16) for groups above 16.
int32_t decode_wave_heads(int32_t n_q_heads, int32_t n_kv_heads);
// Key ranges per group of kv heads the split kernel is launched with (bf16 or FP8 pools, which
// differ in resident workgroups); -1 if too many.
int32_t decode_grid(int32_t batch, int32_t max_seq_len, int32_t n_kv_heads, bool kv8);
size_t decode_workspace(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, bool kv8);
int launch_decode_bf16(const AttnArgs& a, hipStream_t stream);
// Address of the static DECODE scratch array (RAX_DECODE_SCRATCH_BYTES) on the device of
// `stream` (the current device for the null stream), looked up once per device; nullptr if it
// cannot be found.
void* decode_scratch(hipStream_t stream);

// fp32 path (vector ALU; fp32 data, scores formed in double).
int launch_extend_fp32(const AttnArgs& a, hipStream_t stream);
int launch_decode_fp32(const AttnArgs& a, hipStream_t stream);

}  // namespace rax
