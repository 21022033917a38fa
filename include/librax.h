/*
 * librax -- paged-KV attention over a token-granular slot pool, for AMD MI355X (gfx950).
 *
 * The state the calls read and write is the two-level KV memory the SGLang pages describe:
 *
 *   req_to_token[request_row, position] -> slot        ("A walkthrough of SGLang", Main line 4;
 *   k_pool[slot, kv_head, d], v_pool[slot, kv_head, d]   "SGLang" notes, section "KV memory")
 *
 * one slot per token ("Origins: the paper and the first commit", section "Memory: a two-level
 * pool paged by token"). Requests that share a prefix simply hold the same leading slot numbers
 * in their table rows; nothing is copied ("Inside SGLang", Step 3, "Paged KV and the kernels
 * that read it"). Each call handles one layer; the caller indexes layers.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers (HIP device memory), row-major and contiguous,
 *   except where a stride is given. Scalars are host values.
 * - Element format `dtype`: RAX_BF16 (bfloat16, 2 bytes) or RAX_FP32 (4 bytes). K, V, Q and O
 *   of one call share it. Index arrays are int32.
 * - head_dim must be 64 or 128. n_q_heads must be a positive multiple of n_kv_heads; query
 *   head h reads kv head h / (n_q_heads / n_kv_heads) (contiguous groups: grouped-query
 *   attention, "Inside SGLang", Step 3).
 * - Kernels exist for (group G = n_q_heads / n_kv_heads): fp32 EXTEND and DECODE, any G and
 *   head_dim 64 or 128; bf16 EXTEND (plain, ragged and paged) and FP8-pool EXTEND, head_dim 64
 *   or 128, with G from 1 to 256; bf16 (and FP8-pool) DECODE, head_dim 64
 *   or 128 and G from 1 to 256 (above 16, ceil(G / 16) waves per kv head). Any other valid shape
 *   returns RAX_ERR_UNSUPPORTED before anything is enqueued.
 * - `stream` is a hipStream_t (NULL = the null stream). Every call only ENQUEUES work on it:
 *   the library never allocates, frees or synchronises, and keeps no state between calls.
 *   Buffers must stay alive until the stream has passed the call. Calls are thread-safe.
 * - Ownership: the caller owns every buffer, including workspaces.
 * - Errors: a status code is returned (rax_status); no exception crosses the ABI. Arguments
 *   are checked on the host before anything is enqueued, so a call that returns an error has
 *   enqueued nothing. Device-resident values (lengths, slots) cannot be checked on the host:
 *   they must satisfy the contracts stated per call (see each call); kernels clamp lengths to
 *   the host-side maxima so that a violated length contract never indexes past a workspace.
 * - An empty batch (batch == 0, n_new == 0, or total_extend_tokens == 0) returns RAX_OK and
 *   enqueues nothing.
 */
#ifndef LIBRAX_H
#define LIBRAX_H

#include <stddef.h>
#include <stdint.h>

/* The HIP runtime's stream handle. Declared here so that plain C callers need no HIP headers;
 * it is the same type hip_runtime_api.h defines (a repeated identical typedef is valid C11 and
 * C++), so a hipStream_t from the runtime passes unchanged. */
#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t* hipStream_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rax_status {
    RAX_OK = 0,
    RAX_ERR_NULL = 1,        /* a required pointer is NULL                                    */
    RAX_ERR_SHAPE = 2,       /* a size or count is negative, zero where it may not be, or
                                inconsistent with another                                     */
    RAX_ERR_DTYPE = 3,       /* unknown element format                                        */
    RAX_ERR_UNSUPPORTED = 4, /* a valid shape with no kernel in the library (head_dim, group) */
    RAX_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the *_workspace_bytes figure   */
    RAX_ERR_LAUNCH = 6,      /* the HIP runtime refused the launch                            */
    RAX_ERR_SCRATCH = 7      /* the shapes need more than the no-allocation call's static
                                scratch (RAX_DECODE_SCRATCH_BYTES)                             */
} rax_status;

typedef enum rax_dtype {
    RAX_BF16 = 0,
    RAX_FP32 = 1,
    RAX_FP8_E4M3 = 2 /* K/V pool element of the *_fp8 calls (workspace queries only)   */
} rax_dtype;

/* Library version, major * 10000 + minor * 100 + patch. */
int rax_version(void);

/* Static, human-readable name of a status code ("RAX_OK", ...); "unknown status" otherwise. */
const char* rax_status_str(rax_status status);

/*
 * kv_store -- write new K/V rows into pool slots by index.
 *
 * Defined by "Origins: the paper and the first commit", section "Execution: RadixAttention and
 * two sets of kernels": the attention layer writes the layer's freshly computed K and V into
 * the key and value buffers at the batch's output slot locations (out_cache_loc, "A walkthrough
 * of SGLang", Main line 3), before the attention kernel reads the pool.
 *
 *   for i < n_new:  k_pool[loc[i], :, :] = k_new[i, :, :];  v_pool[loc[i], :, :] = v_new[i, :, :]
 *
 * Arguments
 *   dtype        element format of k_new, v_new, k_pool, v_pool.
 *   k_new, v_new [n_new, n_kv_heads, head_dim] rows to write.
 *   loc          [n_new] int32 destination slots. CONTRACT: distinct and in [0, num_slots).
 *                Out-of-range or repeated entries are undefined behaviour (not checked by this
 *                call; rax_check_kv_store counts them).
 *   k_pool, v_pool [num_slots, n_kv_heads, head_dim] pools, written in place. No other row
 *                changes; the copy is bit-exact.
 * Errors: RAX_ERR_NULL, RAX_ERR_SHAPE (n_new < 0, n_new > num_slots, num_slots <= 0,
 *   n_kv_heads <= 0), RAX_ERR_DTYPE, RAX_ERR_UNSUPPORTED (head_dim), RAX_ERR_LAUNCH.
 */
rax_status rax_kv_store(rax_dtype dtype, const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                        void* k_pool, void* v_pool, int64_t num_slots, int32_t n_kv_heads, int32_t head_dim,
                        hipStream_t stream);

/*
 * extend_attention -- EXTEND: the new suffix tokens of each request attend causally to the
 * request's cached prefix and to themselves.
 *
 * Defined by "Origins: the paper and the first commit": self-test answer 2 (only the suffix
 * that missed the prefix cache is computed; attention reads the prefix's cached KV and the KV
 * just computed) and section "Batching: Req, Batch and the three forward modes" (the model
 * input is the suffix only; seq_len = prefix_len + extend_len). Per head the arithmetic is the
 * four steps of "Inside SGLang", Step 3: scores Q K^T, times sm_scale, minus infinity above
 * the causal diagonal, softmax along each row, times V.
 *
 * For request b with r = req_pool_indices[b], p = prefix_lens[b], e = extend_lens[b],
 * s = extend_start_loc[b], suffix row i (0 <= i < e) sits at absolute position p + i and sees
 * the keys at positions 0 .. p + i (bottom-right causal alignment, itself included):
 *
 *   o[s + i, h, :] = softmax_j( sm_scale * q[s + i, h, :] . K[slot_j, h / G, :] ) V[slot_j, h/G, :]
 *   with slot_j = req_to_token[r * r2t_stride + j], j = 0 .. p + i.
 *
 * EVERY key, suffix included, is read from the pool: the caller must rax_kv_store the suffix
 * rows first, on the same stream.
 *
 * Arguments
 *   q, o          [total_extend_tokens, n_q_heads, head_dim]; requests back to back.
 *   k_pool, v_pool [num_slots, n_kv_heads, head_dim].
 *   req_to_token  request table, row stride r2t_stride (int32 elements).
 *   req_pool_indices, prefix_lens, extend_lens, extend_start_loc   [batch] int32 (device).
 *   max_extend_len  >= every extend_lens[b]     (host; sizes the grid)
 *   max_seq_len     >= every p + e, <= r2t_stride (host)
 *   sm_scale      softmax scale applied to the raw score (1/sqrt(head_dim) in the pages).
 *   workspace     scratch of at least rax_extend_workspace_bytes(...) bytes (may be NULL when
 *                 that figure is 0). Over bf16 and FP8 pools (query the *_fp8 calls with
 *                 RAX_FP8_E4M3) the figure is nonzero when the (request, kv head) pairs times
 *                 the row tiles (256 / G suffix tokens each) number at most 128 and
 *                 max_seq_len spans at least 1,024 keys: each row tile's keys are then split
 *                 over S = floor(256 / (pairs x tiles)) <= 16 workgroups whose partial rows (fp32) and log2-sum-exps a second
 *                 kernel merges, S * total_extend_tokens * n_q_heads * (head_dim + 1) * 4 bytes
 *                 (plus alignment). The same holds for the paged and ragged calls. The
 *                 workspace must not be used by other work until the call has passed on the
 *                 stream; the fp32 path needs none. (Split summation order: the results agree
 *                 with the unsplit ones to bf16 rounding, not bit for bit.)
 * Device-side CONTRACT: 0 <= prefix_lens[b], 0 <= extend_lens[b] <= max_extend_len,
 *   prefix_lens[b] + extend_lens[b] <= max_seq_len, extend_start_loc[b] + extend_lens[b] <=
 *   total_extend_tokens, the first p + e entries of each used table row are valid slots.
 *   A request with e = 0 produces no rows.
 * Output rounding: bf16 outputs are fp32 results rounded to nearest even.
 * Errors: RAX_ERR_NULL, RAX_ERR_SHAPE, RAX_ERR_DTYPE, RAX_ERR_UNSUPPORTED, RAX_ERR_WORKSPACE,
 *   RAX_ERR_LAUNCH.
 */
size_t rax_extend_workspace_bytes(rax_dtype dtype, int32_t batch, int64_t total_extend_tokens,
                                  int32_t max_extend_len, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim);

rax_status rax_extend_attention(rax_dtype dtype, const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                const int32_t* extend_lens, const int32_t* extend_start_loc, int32_t batch,
                                int64_t total_extend_tokens, int32_t max_extend_len, int32_t max_seq_len,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * extend_attention_ragged -- EXTEND with the suffix K/V taken straight from the just-computed
 * rows, optionally storing them into the pool in the same call.
 *
 * The pages describe attention over "the prefix's cached KV together with the KV just
 * computed" ("Origins...", self-test answer 2) and a ragged kernel for the new tokens beside a
 * paged kernel for the cached prefix ("Inside SGLang", Step 3). Same result as kv_store then
 * rax_extend_attention (the stored values are the same bits), with:
 *
 *   key position j < p        : K/V[req_to_token[r * r2t_stride + j], h / G, :] (the pool)
 *   key position j = p + i    : k_new / v_new[extend_start_loc[b] + i, h / G, :]
 *
 * Arguments (others as rax_extend_attention)
 *   k_new, v_new  [total_extend_tokens, n_kv_heads, head_dim], rows in the order of q (the
 *                 suffix rows of every request, back to back). Read only.
 *   store_loc     NULL, or [total_extend_tokens] int32 (device): when given, new row t is also
 *                 written to pool slot store_loc[t] (the bf16 kernel stores inside the
 *                 attention kernel; fp32 launches the copy first). The pools are written only
 *                 then.
 * Device-side CONTRACT: only the first p entries of each used table row are read as slots;
 *   store_loc entries are distinct, inside the pool, and not among any request's prefix slots.
 * Errors: as rax_extend_attention; RAX_ERR_NULL when k_new or v_new is NULL.
 */
rax_status rax_extend_attention_ragged(rax_dtype dtype, const void* q, void* o, const void* k_new,
                                       const void* v_new, const int32_t* store_loc, void* k_pool,
                                       void* v_pool, int64_t num_slots, const int32_t* req_to_token,
                                       int64_t r2t_stride, const int32_t* req_pool_indices,
                                       const int32_t* prefix_lens, const int32_t* extend_lens,
                                       const int32_t* extend_start_loc, int32_t batch,
                                       int64_t total_extend_tokens, int32_t max_extend_len,
                                       int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, float sm_scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * decode_attention -- DECODE: one query per request over its whole context.
 *
 * Defined by "Inside SGLang", Step 3, "Prefill and decode have different shapes": each request
 * has one new query whose score row is 1 x n over every earlier token, read from the slots its
 * table row names ("Paged KV and the kernels that read it": one query against many scattered
 * slots). The current token's K/V must already be stored (one slot per request per step,
 * "Origins...", "Batching"). No mask applies.
 *
 *   o[b, h, :] = softmax_j( sm_scale * q[b, h, :] . K[slot_j, h / G, :] ) V[slot_j, h / G, :],
 *   slot_j = req_to_token[req_pool_indices[b] * r2t_stride + j], j = 0 .. seq_lens[b] - 1.
 *
 * The work is split along the keys (split-K) in a balanced way: a plan lays the
 * requests' contexts end to end (each rounded up to a multiple of 64 keys) and cuts that
 * stream into equal ranges of 256..4096 keys, one per workgroup, so that every workgroup moves
 * the same bytes whatever the mix of context lengths. Partial results (fp32 o and a
 * log-sum-exp per request and range) go to the workspace and a merge kernel combines them.
 * The kernels run on `stream` in order: split (which computes the plan itself for batches up
 * to 1,024 requests; larger batches get a separate plan kernel first), then merge. The
 * workspace holds the plan and the partials and must not be used by other work until they
 * have run.
 *
 * Arguments
 *   q, o          [batch, n_q_heads, head_dim].
 *   seq_lens      [batch] int32 (device). CONTRACT: 1 <= seq_lens[b] <= max_seq_len.
 *                 A request with seq_lens[b] <= 0 gets an all-zero output row.
 *   max_seq_len   host bound, <= r2t_stride.
 *   workspace     at least rax_decode_workspace_bytes(...) bytes.
 * Errors: as extend_attention.
 */
size_t rax_decode_workspace_bytes(rax_dtype dtype, int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim);

rax_status rax_decode_attention(rax_dtype dtype, const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                float sm_scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * decode_attention_noalloc -- rax_decode_attention with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * The plan and the partials that rax_decode_attention keeps in the caller's workspace live
 * instead in a static device array of RAX_DECODE_SCRATCH_BYTES inside the library; each GPU the
 * library runs on holds its own copy until the process ends. The call allocates and frees
 * nothing. Its first call on a device looks up that device's copy (not a stream operation:
 * make the first call outside graph capture). Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents; nothing in it needs to start at any value. Calls that
 * overlap on one GPU (on different streams, or from different threads, until the stream has
 * passed the call) race on the array: serialise them. Arguments, kernels and results are those
 * of rax_decode_attention (the same bits).
 *
 * Errors: as rax_decode_attention; RAX_ERR_SCRATCH when rax_decode_workspace_bytes(dtype, ...)
 *   of these shapes exceeds RAX_DECODE_SCRATCH_BYTES (for example 64 requests of up to 4,096
 *   keys with 32 q / 8 kv heads and head_dim 128 need 7.1 MiB, 128 requests of up to 8,192
 *   keys 8.1 MiB, 8 requests of up to 131,072 keys with 64 q heads 12.3 MiB; 1,000 requests of
 *   up to 8,192 keys with 32 q heads need 47 MiB and are refused); RAX_ERR_LAUNCH when the
 *   array cannot be found on the stream's device.
 */
#define RAX_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

rax_status rax_decode_attention_noalloc(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                        const void* v_pool, int64_t num_slots,
                                        const int32_t* req_to_token, int64_t r2t_stride,
                                        const int32_t* req_pool_indices, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                        hipStream_t stream);

/*
 * Page tables -- the same EXTEND and DECODE over a pool allocated in pages of P slots ("A
 * walkthrough of SGLang", Exercises, exercise 2: the page-size option allocates and matches by
 * pages of, e.g., 16, 32 or 64 tokens; the first version used one slot per token, "Origins:
 * the paper and the first commit"). The request table then names one page per P positions:
 *
 *   slot of position j of table row r = page_table[r * pt_stride + j / P] * P + j % P
 *
 * (page k of a request holds its positions kP .. kP + P - 1 in order). Everything else --
 * layouts, lengths, workspace (rax_extend/decode_workspace_bytes), outputs -- is as in the
 * token-granular calls; with P = 1 the page table is a token table and the result is that
 * of rax_extend_attention / rax_decode_attention.
 *
 * Arguments
 *   page_table    int32 (device), row stride pt_stride entries; pt_stride * P >= max_seq_len.
 *   page_size     P, a power of two from 1 to 2^20 (else RAX_ERR_SHAPE).
 * Device-side CONTRACT: the entries for positions 0 .. L-1 of each used row are pages with
 *   page * P + P <= num_slots. bf16 (MFMA kernels) and fp32; FP8 pools through
 *   rax_extend_attention_paged_fp8 / rax_decode_attention_paged_fp8 (below).
 */
rax_status rax_extend_attention_paged(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                      const void* v_pool, int64_t num_slots, const int32_t* page_table,
                                      int64_t pt_stride, int32_t page_size,
                                      const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                      const int32_t* extend_lens, const int32_t* extend_start_loc,
                                      int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                      int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, float sm_scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

rax_status rax_decode_attention_paged(rax_dtype dtype, const void* q, void* o, const void* k_pool,
                                      const void* v_pool, int64_t num_slots, const int32_t* page_table,
                                      int64_t pt_stride, int32_t page_size,
                                      const int32_t* req_pool_indices, const int32_t* seq_lens,
                                      int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, float sm_scale,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 KV pools -- the K and V pools hold one OCP FP8 E4M3 byte per element (no infinities; NaN
 * only at 0x7F/0xFF; largest finite magnitude 448), and an element's value is
 * scale * e4m3(byte) with one float scale per pool ("Inside SGLang", Step 6: with an FP8 KV
 * cache every token costs half the bytes, attention reads the FP8 cache without a separate
 * dequantisation pass, and a scale that the checkpoint does not provide is 1.0). Q, O and the
 * new K/V rows given to the store stay bf16. Pools are uint8 [num_slots, n_kv_heads, head_dim];
 * everything else as in the bf16 calls. Scales must be finite and > 0 (else RAX_ERR_SHAPE).
 *
 * rax_kv_store_fp8 -- as rax_kv_store, but each new bf16 element x is written as the E4M3 byte
 *   nearest to clamp(float32(x) * r, -448, 448), ties to the even code, where r is 1/scale
 *   computed in double and rounded once to float. Inputs must be finite (NaN inputs give an
 *   undefined byte). Same loc contract as rax_kv_store.
 *
 * rax_extend_attention_fp8 -- rax_extend_attention over FP8 pools (the same head_dims and
 *   group sizes as bf16): the scores use k_scale * e4m3(K) and the values v_scale * e4m3(V).
 *   The kernel stages the E4M3 tiles in LDS, widens them to bf16 (exact) and applies k_scale to
 *   the scores and v_scale to the output. Workspace: rax_extend_workspace_bytes(RAX_FP8_E4M3,
 *   ...) (the key splits' partials, as for bf16 pools; NULL is accepted when it is 0).
 *
 * rax_decode_attention_fp8 -- rax_decode_attention over FP8 pools: the scores use
 *   k_scale * e4m3(K) and the values v_scale * e4m3(V). Every E4M3 value is exactly a bf16
 *   value, so the kernel widens the bytes in registers and applies k_scale to the scores and
 *   v_scale to the output. Workspace: rax_decode_workspace_bytes(RAX_FP8_E4M3, ...).
 */
rax_status rax_kv_store_fp8(const void* k_new, const void* v_new, const int32_t* loc, int64_t n_new,
                            void* k_pool, void* v_pool, int64_t num_slots, int32_t n_kv_heads,
                            int32_t head_dim, float k_scale, float v_scale, hipStream_t stream);

rax_status rax_extend_attention_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                    int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                    const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                    const int32_t* extend_lens, const int32_t* extend_start_loc,
                                    int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                    int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

rax_status rax_decode_attention_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                    int64_t num_slots, const int32_t* req_to_token, int64_t r2t_stride,
                                    const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                                    int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rax_extend_attention_ragged_paged -- rax_extend_attention_ragged with the cached prefix read
 * through a page table (page_table, pt_stride, page_size as in rax_extend_attention_paged):
 * suffix positions come from k_new / v_new, prefix positions from the pool slots the page table
 * names, and store_loc (optional) still names one token slot per suffix row. The ragged kernel
 * beside a paged one that "Inside SGLang", Step 3 describes, over the paged pool of "A
 * walkthrough of SGLang", Exercises, exercise 2. Device-side CONTRACT: the page entries that
 * cover positions 0 .. p-1 of each used row are pages inside the pool (later entries of the
 * row are not used as pages); store_loc as in rax_extend_attention_ragged. Same errors as both
 * calls.
 */
rax_status rax_extend_attention_ragged_paged(rax_dtype dtype, const void* q, void* o, const void* k_new,
                                             const void* v_new, const int32_t* store_loc, void* k_pool,
                                             void* v_pool, int64_t num_slots, const int32_t* page_table,
                                             int64_t pt_stride, int32_t page_size,
                                             const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                             const int32_t* extend_lens, const int32_t* extend_start_loc,
                                             int32_t batch, int64_t total_extend_tokens, int32_t max_extend_len,
                                             int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, float sm_scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/*
 * rax_extend_attention_paged_fp8, rax_decode_attention_paged_fp8 -- the FP8-pool calls above
 * with a page table of page_size slots per page in place of the token table: the arguments of
 * rax_extend_attention_fp8 / rax_decode_attention_fp8 with (page_table, pt_stride, page_size)
 * as in rax_extend_attention_paged, and the same scales, contract and errors (a page size that
 * is not a power of two from 1 to 2^20 gives RAX_ERR_SHAPE). The two options of the pages
 * together: pages of P slots ("A walkthrough of SGLang", Exercises, exercise 2) over an FP8
 * cache ("Inside SGLang", Step 6).
 */
rax_status rax_extend_attention_paged_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                          int64_t num_slots, const int32_t* page_table, int64_t pt_stride,
                                          int32_t page_size, const int32_t* req_pool_indices,
                                          const int32_t* prefix_lens, const int32_t* extend_lens,
                                          const int32_t* extend_start_loc, int32_t batch,
                                          int64_t total_extend_tokens, int32_t max_extend_len,
                                          int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);

rax_status rax_decode_attention_paged_fp8(const void* q, void* o, const void* k_pool, const void* v_pool,
                                          int64_t num_slots, const int32_t* page_table, int64_t pt_stride,
                                          int32_t page_size, const int32_t* req_pool_indices,
                                          const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                          float sm_scale, float k_scale, float v_scale, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* Number of key ranges per group of kv heads that rax_decode_attention launches for these
 * shapes (bf16; 1 for fp32 or empty shapes; -1 if the shapes need more than 2^31 - 1). Ranges
 * past the end of the actual key stream exit at once. For tests and reports. With more than
 * 16 query heads per kv head, pass n_kv_heads * ceil(G / 16) (the waves per range). */
int32_t rax_decode_num_splits(rax_dtype dtype, int32_t batch, int32_t max_seq_len, int32_t n_kv_heads);

/*
 * Debug checks of the device-side contracts -- for callers that want the contracts above
 * verified (the attention and store calls themselves trust their index arrays).
 *
 * Each check enqueues kernels on `stream` that read the index arrays a call would be given,
 * only inside the bounds of the host arguments (never through an index that fails its check),
 * and writes to `counts` (device int32[RAX_CHECK_COUNT], zeroed by the check itself) the number
 * of entries that break each contract:
 *
 *   RAX_CHECK_LENGTH     requests whose lengths or start break the call's CONTRACT (EXTEND:
 *                        0 <= p, 0 <= e <= max_extend_len, p + e <= max_seq_len, 0 <= s,
 *                        s + e <= total_extend_tokens; DECODE: seq_lens[b] <= max_seq_len);
 *                        their positions are not examined further.
 *   RAX_CHECK_ROW        requests with valid lengths that read keys, whose
 *                        req_pool_indices[b] lies outside [0, table_rows); their positions are
 *                        not examined further.
 *   RAX_CHECK_SLOT       positions the call reads whose slot (token table) or page (page
 *                        table: page * P + P <= num_slots) lies outside the pool; for the
 *                        store checks, loc / store_loc entries outside [0, num_slots).
 *   RAX_CHECK_DUPLICATE  loc / store_loc entries equal to an earlier entry.
 *   RAX_CHECK_OVERLAP    positions a ragged call reads from the pool whose slot is also one
 *                        of its store_loc slots.
 *
 * The positions a call reads: EXTEND 0 .. p + e - 1 (0 .. p - 1 for the ragged call), for
 * requests with e > 0; DECODE 0 .. seq_lens[b] - 1. All zero means the arrays satisfy the
 * contracts the checks cover. Counts are per entry and wrap past 2^31 - 1.
 *
 * Arguments (as the call being checked, plus)
 *   table_rows   rows of req_to_token / page_table (stride table_stride entries).
 *   page_size    1 for a token table, else the page size (a power of two up to 2^20).
 *   workspace    the duplicate and overlap checks' bitmap, rax_check_workspace_bytes(num_slots)
 *                bytes: needed by rax_check_kv_store, and by rax_check_extend when store_loc is
 *                given; contents are overwritten.
 *   counts       device int32[RAX_CHECK_COUNT], written by the check.
 * Errors: RAX_ERR_NULL, RAX_ERR_SHAPE (as the checked call, plus page_size, table_rows <= 0
 *   with batch > 0, max_seq_len > table_stride * page_size, store_loc without ragged),
 *   RAX_ERR_WORKSPACE, RAX_ERR_LAUNCH. Like every call they only enqueue work: read `counts`
 *   after the stream has passed them.
 */
typedef enum rax_check_item {
    RAX_CHECK_LENGTH = 0,
    RAX_CHECK_ROW = 1,
    RAX_CHECK_SLOT = 2,
    RAX_CHECK_DUPLICATE = 3,
    RAX_CHECK_OVERLAP = 4,
    RAX_CHECK_COUNT = 5
} rax_check_item;

size_t rax_check_workspace_bytes(int64_t num_slots);

rax_status rax_check_kv_store(const int32_t* loc, int64_t n_new, int64_t num_slots, void* workspace,
                              size_t workspace_bytes, int32_t* counts, hipStream_t stream);

rax_status rax_check_extend(const int32_t* table, int64_t table_rows, int64_t table_stride,
                            int32_t page_size, const int32_t* req_pool_indices, const int32_t* prefix_lens,
                            const int32_t* extend_lens, const int32_t* extend_start_loc, int32_t batch,
                            int64_t total_extend_tokens, int32_t max_extend_len, int32_t max_seq_len,
                            int64_t num_slots, int32_t ragged, const int32_t* store_loc, void* workspace,
                            size_t workspace_bytes, int32_t* counts, hipStream_t stream);

rax_status rax_check_decode(const int32_t* table, int64_t table_rows, int64_t table_stride,
                            int32_t page_size, const int32_t* req_pool_indices, const int32_t* seq_lens,
                            int32_t batch, int32_t max_seq_len, int64_t num_slots, int32_t* counts,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBRAX_H */
