// EXTEND attention, bf16, head_dim 128: new suffix rows attend causally to the request's cached
// prefix and to themselves, every key gathered from the slot pool through req_to_token.
//
// With a prefix cache only the missed suffix is computed, and attention reads the prefix's
// cached KV together with the KV just computed ("Origins: the paper and the first commit",
// self-test answer 2 and "Batching: Req, Batch and the three forward modes"). Per head the
// arithmetic is "Inside SGLang", Step 3: Q K^T, scale, -inf above the (bottom-right) causal
// diagonal, row softmax, times V. Evaluated blockwise with an online softmax (running max and
// sum per row), which is an exact reformulation of the row softmax.
//
// Design (gfx950, wave64, 256 threads = 4 waves per workgroup):
//  * Work item: (request b, kv head g, BM = 128 query rows). The rows are (token, head) pairs
//    of the G query heads sharing kv head g, token-major, so one gathered K/V tile feeds
//    128 / G tokens x G heads. Each wave owns 32 rows.
//  * Key tiles of 64: 256 threads gather the 64 K rows and 64 V rows (256 B per kv head per
//    row, 16-byte loads, 16 lanes per row: coalesced). Slot numbers are loaded two tiles
//    ahead and rows one tile ahead, so the dependent slot -> row load pair never stalls the
//    MFMAs. Two LDS buffers, one barrier per tile. K and V are both stored row-major, XOR-
//    swizzled in 16-byte units so that the operand reads and the stores avoid bank conflicts.
//  * S^T = K Q^T with 32x32x16 bf16 MFMAs: keys are the M dimension (read from LDS), query
//    rows the N dimension (Q stays in registers for the whole key loop). The C layout puts
//    one query row per lane column, so the row max/sum are per lane plus one exchange with
//    the other half-wave.
//  * O^T = V^T P^T, also 32x32x16: P^T is the score C fragment converted to bf16 in place, so
//    P never leaves registers. The V^T operand comes from the row-major V tile through the
//    gfx950 transposed LDS read (ds_read_b64_tr_b16), in the key order the P^T fragment has.
//  * Softmax: sm_scale * log2(e) is folded into one FMA before exp2; the accumulators are only
//    rescaled when a row max grows by more than 2^8 (exact: P and the row sum share the
//    reference max).
//  * Causal mask only on the tiles that cross the diagonal (a separate loop, so full tiles run
//    no mask code); keys past the last visible key of the workgroup reuse a valid slot and are
//    masked, so no load leaves the request's slots.
//  * Pool addressing: a per-kv-head base pointer (uniform, in SGPRs) plus a 32-bit byte offset
//    slot * row_bytes (24-bit multiply) when the pool fits (slots * row_bytes <= 2^32, e.g. the
//    2,097,152-slot, 8-head pool of exactly 4 GiB); 64-bit arithmetic otherwise.
//  * Workgroup order is XCD-aware: consecutive workgroup ids go to different XCDs, so the
//    linear id is remapped so that all tiles of one (request, kv head) run on one XCD and
//    share its L2 for the gathered K/V; the longest (last) tiles start first.
#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

namespace {

constexpr int kExtD = 128;
constexpr int kExtBM = 128;
constexpr int kExtBN = 64;
constexpr int kExtThreads = 256;
constexpr int kXcds = 8;

// In units of 2^kLazyLog2, how far a row max may rise before the accumulators are rescaled.
constexpr float kLazyLog2 = 8.f;

// LDS swizzles of 16-byte units within a 256-byte row (valid for 32- or 64-bank LDS).
//  K: unit ^ (key & 15): the 16 consecutive rows that one 16-lane phase of an MFMA operand
//     read touches land on 16 distinct units.
//  V: bit 3 of the unit is toggled by bit 1 (the head_dim half a 16-lane group reads), then
//     ^ 2 (key & 3): the four rows of one transposed read (keys 4n .. 4n+3, two units each)
//     land on eight distinct units, and the two 16-lane groups of a half-wave on the other
//     eight. Stores write whole rows, so any permutation within a row is conflict-free.
__device__ __forceinline__ int swz_k(int key, int unit) { return unit ^ (key & 15); }
__device__ __forceinline__ int swz_v(int key, int unit) {
    return (unit ^ (((unit >> 1) & 1) << 3)) ^ (2 * (key & 3));
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group, lane 4j + c
// supplies the address of four 16-bit values; lane i receives value i % 4 of the chunk of lane
// 4j + i / 4, for j = 0..3.
__device__ __forceinline__ uint2 ds_read_tr16_b64(const char* lds_addr) {
    typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_addr));
    return __builtin_bit_cast(uint2, v);
}

// 16 bytes at byte offset slot * row_bytes + off from a uniform base.
template <bool OFF32>
__device__ __forceinline__ uint4 pool_load(const char* base, int slot, uint32_t row_bytes, uint32_t off) {
    if constexpr (OFF32) {
        return *(const uint4*)(base + (__umul24((uint32_t)slot, row_bytes) + off));
    } else {
        return *(const uint4*)(base + ((uint64_t)(uint32_t)slot * row_bytes + off));
    }
}

template <int G, bool OFF32>
__global__ __launch_bounds__(kExtThreads, 2) void extend_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ extend_start_loc,
    int64_t total_tokens, int32_t max_extend_len, int32_t max_seq_len, int32_t Hq, int32_t Hkv,
    int32_t batch, int32_t tiles, float scale_log2) {
    constexpr int D = kExtD;
    constexpr int BQ = kExtBM / G;  // tokens per workgroup

    // Two LDS buffers, each a 64-key tile of K and V, row-major [key][16 units of 8 bf16].
    __shared__ uint4 k_lds[2][kExtBN * 16];
    __shared__ uint4 v_lds[2][kExtBN * 16];

    // ---- workgroup -> (pair = b * Hkv + g, tile), XCD-aware
    const int pairs = batch * Hkv;
    const int xcd = blockIdx.x % kXcds;
    const int k = blockIdx.x / kXcds;
    const int pair = xcd + kXcds * (k / tiles);
    if (pair >= pairs) return;
    const int tq = tiles - 1 - (k % tiles);
    const int b = pair / Hkv;
    const int g = pair - b * Hkv;

    const int p = prefix_lens[b];
    int e = min(extend_lens[b], max_extend_len);
    const int s0 = extend_start_loc[b];
    e = (int)min((int64_t)e, total_tokens - s0);
    const int t0 = tq * BQ;
    if (t0 >= e) return;
    const int t_last = min(t0 + BQ, e) - 1;
    const int kend = min(p + t_last + 1, max_seq_len);  // keys 0 .. kend-1 are visible to someone
    const int32_t* row = r2t + (int64_t)rpi[b] * r2t_stride;
    const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
    const char* kbase = (const char*)k_pool + (int64_t)g * D * 2;
    const char* vbase = (const char*)v_pool + (int64_t)g * D * 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;  // query row within the wave (MFMA N index)
    const int h2 = lane >> 5;   // k-group of the MFMA operands

    // ---- this lane's query row
    const int r = 32 * wave + col;
    const int t = t0 + r / G;
    const int hl = r % G;
    const bool row_ok = t < e;
    const int t_ld = row_ok ? t : e - 1;
    const int64_t qo_row = ((int64_t)(s0 + t_ld) * Hq + (int64_t)g * G + hl) * D;
    bf16x8 qop[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = as_bf16x8(*(const uint4*)(q + qo_row + 16 * s + 8 * h2));

    // ---- cooperative gather: thread (seg, grp) moves 16-byte unit `seg` of keys grp + 16 i
    const int seg = tid & 15;
    const int grp = tid >> 4;
    const uint32_t seg_off = 16u * seg;
    const int ntiles = (kend + kExtBN - 1) / kExtBN;
    int slot0, slot1, slot2, slot3;
    uint4 kst0, kst1, kst2, kst3, vst0, vst1, vst2, vst3;
#define RAX_LOAD_SLOTS(TILE)                                                                \
    {                                                                                       \
        const int kb_ = (TILE) * kExtBN + grp;                                              \
        slot0 = row[min(kb_, kend - 1)];                                                    \
        slot1 = row[min(kb_ + 16, kend - 1)];                                               \
        slot2 = row[min(kb_ + 32, kend - 1)];                                               \
        slot3 = row[min(kb_ + 48, kend - 1)];                                               \
    }
#define RAX_GATHER()                                                                        \
    {                                                                                       \
        kst0 = pool_load<OFF32>(kbase, slot0, row_bytes, seg_off);                          \
        vst0 = pool_load<OFF32>(vbase, slot0, row_bytes, seg_off);                          \
        kst1 = pool_load<OFF32>(kbase, slot1, row_bytes, seg_off);                          \
        vst1 = pool_load<OFF32>(vbase, slot1, row_bytes, seg_off);                          \
        kst2 = pool_load<OFF32>(kbase, slot2, row_bytes, seg_off);                          \
        vst2 = pool_load<OFF32>(vbase, slot2, row_bytes, seg_off);                          \
        kst3 = pool_load<OFF32>(kbase, slot3, row_bytes, seg_off);                          \
        vst3 = pool_load<OFF32>(vbase, slot3, row_bytes, seg_off);                          \
    }
#define RAX_TO_LDS(BUF)                                                                     \
    {                                                                                       \
        uint4* kl_ = k_lds[BUF];                                                            \
        uint4* vl_ = v_lds[BUF];                                                            \
        kl_[(grp + 0) * 16 + swz_k(grp + 0, seg)] = kst0;                                   \
        vl_[(grp + 0) * 16 + swz_v(grp + 0, seg)] = vst0;                                   \
        kl_[(grp + 16) * 16 + swz_k(grp + 16, seg)] = kst1;                                 \
        vl_[(grp + 16) * 16 + swz_v(grp + 16, seg)] = vst1;                                 \
        kl_[(grp + 32) * 16 + swz_k(grp + 32, seg)] = kst2;                                 \
        vl_[(grp + 32) * 16 + swz_v(grp + 32, seg)] = vst2;                                 \
        kl_[(grp + 48) * 16 + swz_k(grp + 48, seg)] = kst3;                                 \
        vl_[(grp + 48) * 16 + swz_v(grp + 48, seg)] = vst3;                                 \
    }

    // ---- per-lane constants of the transposed V reads: 16-lane group gi holds head_dim half
    // dh = gi & 1 and k-group h2; lane i16 = 4 jr + cc reads key offset jr and head_dim
    // 4 cc .. 4 cc + 3 of that half.
    const int i16 = lane & 15;
    const int dh = (lane >> 4) & 1;
    const int jr = i16 >> 2;
    const int cc = i16 & 3;

    float m = -INFINITY;
    float lsum = 0.f;
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    const int last_q = p + t;  // last key position this row may see
    // Tiles 0 .. n_full-1 hold only keys <= p + t0, visible to every row of the workgroup.
    const int n_full = min(ntiles, (p + t0 + 1) / kExtBN);

    // One 64-key tile: stage the next tile, scores, (mask), softmax, P V.
#define RAX_TILE(MASK)                                                                      \
    {                                                                                       \
        const int buf = it & 1;                                                             \
        const int j0 = it * kExtBN;                                                         \
        __syncthreads(); /* tile `it` is complete in `buf`; the other buffer is free */     \
        if (it + 1 < ntiles) RAX_TO_LDS(buf ^ 1)                                            \
        if (it + 2 < ntiles) {                                                              \
            RAX_GATHER()                                                                    \
            if (it + 3 < ntiles) RAX_LOAD_SLOTS(it + 3)                                     \
        }                                                                                   \
        f32x16 st[2];                                                                       \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                                  \
            _Pragma("unroll") for (int i = 0; i < 16; ++i) st[mb][i] = 0.f;                 \
            const int key = 32 * mb + col;                                                  \
            _Pragma("unroll") for (int s = 0; s < D / 16; ++s) {                            \
                const uint4 a = k_lds[buf][key * 16 + swz_k(key, 2 * s + h2)];              \
                st[mb] = mfma32x32x16(as_bf16x8(a), qop[s], st[mb]);                        \
            }                                                                               \
        }                                                                                   \
        if (MASK) {                                                                         \
            _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                \
            _Pragma("unroll") for (int jj = 0; jj < 4; ++jj)                                \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                 \
                if (j0 + 32 * mb + 8 * jj + 4 * h2 + i > last_q) st[mb][4 * jj + i] = -INFINITY; \
            }                                                                               \
        }                                                                                   \
        float mx = -INFINITY;                                                               \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                    \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[mb][i]);           \
        mx = wave_max_xor(mx, 32) * scale_log2;                                             \
        if (__any(mx > m + kLazyLog2)) {                                                    \
            const float m_new = fmaxf(m, mx);                                               \
            const float alpha = fast_exp2(m - m_new);                                       \
            m = m_new;                                                                      \
            lsum *= alpha;                                                                  \
            _Pragma("unroll") for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;         \
        }                                                                                   \
        uint4 pf[4];                                                                        \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                  \
            float pv[8];                                                                    \
            _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                 \
                pv[j] = fast_exp2(fmaf(st[kk >> 1][8 * (kk & 1) + j], scale_log2, -m));     \
                lsum += pv[j];                                                              \
            }                                                                               \
            pf[kk].x = pack_bf16x2(pv[0], pv[1]);                                           \
            pf[kk].y = pack_bf16x2(pv[2], pv[3]);                                           \
            pf[kk].z = pack_bf16x2(pv[4], pv[5]);                                           \
            pf[kk].w = pack_bf16x2(pv[6], pv[7]);                                           \
        }                                                                                   \
        const char* vb = (const char*)v_lds[buf];                                           \
        _Pragma("unroll") for (int dt = 0; dt < D / 32; ++dt) {                             \
            const int unit = 4 * dt + 2 * dh + (cc >> 1);                                   \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                              \
                const int key0 = 16 * kk + 4 * h2 + jr;                                     \
                const uint2 h0 = ds_read_tr16_b64(vb + key0 * 256 + swz_v(key0, unit) * 16 + 8 * (cc & 1)); \
                const int key1 = key0 + 8;                                                  \
                const uint2 h1 = ds_read_tr16_b64(vb + key1 * 256 + swz_v(key1, unit) * 16 + 8 * (cc & 1)); \
                const uint4 av = make_uint4(h0.x, h0.y, h1.x, h1.y);                        \
                acc[dt] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pf[kk]), acc[dt]);          \
            }                                                                               \
        }                                                                                   \
    }

    // prologue: tile 0 in LDS buffer 0, tile 1 in registers, slots of tile 2 in registers
    RAX_LOAD_SLOTS(0)
    RAX_GATHER()
    RAX_TO_LDS(0)
    if (ntiles > 1) {
        RAX_LOAD_SLOTS(1)
        RAX_GATHER()
    }
    if (ntiles > 2) RAX_LOAD_SLOTS(2)

    int it = 0;
    for (; it < n_full; ++it) RAX_TILE(false)
    for (; it < ntiles; ++it) RAX_TILE(true)

    lsum += __shfl_xor(lsum, 32, kWave);
    if (row_ok) {
        const float inv = 1.f / lsum;
        uint16_t* orow = o + qo_row;
        // acc[dt][4 jj + i] is head_dim 32 dt + 8 jj + 4 h2 + i
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint2 w;
                w.x = pack_bf16x2(acc[dt][4 * jj + 0] * inv, acc[dt][4 * jj + 1] * inv);
                w.y = pack_bf16x2(acc[dt][4 * jj + 2] * inv, acc[dt][4 * jj + 3] * inv);
                *(uint2*)(orow + 32 * dt + 8 * jj + 4 * h2) = w;
            }
    }
}
#undef RAX_LOAD_SLOTS
#undef RAX_GATHER
#undef RAX_TO_LDS
#undef RAX_TILE

template <int G, bool OFF32>
int launch_g(const AttnArgs& a, hipStream_t stream) {
    constexpr int BQ = kExtBM / G;
    const int tiles = (a.max_extend_len + BQ - 1) / BQ;
    const int pairs = a.batch * a.n_kv_heads;
    const int64_t blocks = (int64_t)((pairs + kXcds - 1) / kXcds) * kXcds * tiles;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL((extend_kernel<G, OFF32>), dim3((unsigned)blocks), dim3(kExtThreads), 0, stream,
                       (const uint16_t*)a.q, (uint16_t*)a.o, (const uint16_t*)a.k_pool,
                       (const uint16_t*)a.v_pool, a.r2t, a.r2t_stride, a.req_pool_indices,
                       a.prefix_lens, a.extend_lens, a.extend_start_loc, a.total_tokens,
                       a.max_extend_len, a.max_seq_len, a.n_q_heads, a.n_kv_heads, a.batch, tiles,
                       a.sm_scale * kLog2e);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int G>
int launch_g(const AttnArgs& a, hipStream_t stream) {
    return pool_fits_32bit_offsets(a.num_slots, a.n_kv_heads, a.head_dim, 2)
               ? launch_g<G, true>(a, stream)
               : launch_g<G, false>(a, stream);
}

}  // namespace

bool extend_bf16_supported(int32_t group, int32_t head_dim) {
    return head_dim == 128 && (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

int launch_extend_bf16(const AttnArgs& a, hipStream_t stream) {
    switch (a.n_q_heads / a.n_kv_heads) {
        case 1: return launch_g<1>(a, stream);
        case 2: return launch_g<2>(a, stream);
        case 4: return launch_g<4>(a, stream);
        case 8: return launch_g<8>(a, stream);
        case 16: return launch_g<16>(a, stream);
        default: return -1;
    }
}

}  // namespace rax
