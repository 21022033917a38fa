// EXTEND attention, bf16, head_dim 64 or 128: new suffix rows attend causally to the request's cached
// prefix and to themselves, every key gathered from the slot pool through req_to_token.
//
// With a prefix cache only the missed suffix is computed, and attention reads the prefix's
// cached KV together with the KV just computed ("Origins: the paper and the first commit",
// self-test answer 2 and "Batching: Req, Batch and the three forward modes"). Per head the
// arithmetic is "Inside SGLang", Step 3: Q K^T, scale, -inf above the (bottom-right) causal
// diagonal, row softmax, times V. Evaluated blockwise with an online softmax (running max and
// sum per row), which is an exact reformulation of the row softmax.
//
// Design (gfx950, wave64, 512 threads = 8 waves per workgroup, one workgroup per CU):
//  * Work item: (request b, kv head g, BM = 256 query rows). The rows are (token, head) pairs
//    of the G query heads sharing kv head g, token-major, so one gathered K/V tile feeds
//    256 / G tokens x G heads (floor(256 / G) tokens when G does not divide 256; the rows past
//    them are idle). Each wave owns 32 rows. Every workgroup reads the whole visible
//    context once, so the K/V traffic is (query rows / 256) x context: the row count per
//    workgroup is what keeps the kernel off the memory roofline.
//  * Key tiles of 64 rows (256 B per kv head per row; head_dim 64 fills half of each LDS row)
//    are copied HBM -> LDS without registers, 16 B per lane (buffer_load_dwordx4 ... lds
//    through a buffer resource when the pool's byte offsets fit 32 bits, the gfx950
//    global_load_lds_dwordx4 otherwise), each lane fetching the unit that the LDS swizzle
//    stores at its destination. Four LDS buffers: tile i is consumed while
//    tiles i+1 and i+2 are in flight, and tile i-1's V is still read (ping-pong, below);
//    slot numbers are loaded one tile before their copy. The buffers are separate LDS objects
//    and the loop is unrolled by four, so every read names its buffer and the compiler does
//    not wait on copies into the other buffers. Before each barrier the wave waits (vmcnt)
//    only for the copies of the tile it is about to read.
//  * Ping-pong: the per-tile barrier would keep the two waves of a SIMD (w and w + 4) in the
//    same phase, both issuing MFMAs, then both the softmax. Waves 4-7 therefore lag by half a
//    tile: in iteration i they run the softmax and P V of tile i-1, then the scores of tile i,
//    while waves 0-3 run tile i whole; each SIMD's MFMA pipe then meets the other wave's
//    softmax for two thirds of the iteration (+2 to +8% measured).
//  * FP8 pools: E4M3 tiles go through two staging buffers per operand (the four bf16 tiles
//    plus 32 KB of staging fill the 160 KB of LDS) and are widened to the bf16 tiles by the
//    lane that copied them, between the two halves of the ping-pong; the compute is the same.
//  * S^T = K Q^T with 32x32x16 bf16 MFMAs: keys are the M dimension (read from LDS), query
//    rows the N dimension (Q stays in registers for the whole key loop). The C layout puts
//    one query row per lane column, so the row max/sum are per lane plus one exchange with
//    the other half-wave.
//  * O^T = V^T P^T, also 32x32x16: P^T is the score C fragment converted to bf16 in place, so
//    P never leaves registers. The V^T operand comes from the row-major V tile through the
//    gfx950 transposed LDS read (ds_read_b64_tr_b16), in the key order the P^T fragment has.
//  * Softmax: sm_scale * log2(e) is folded into one FMA before exp2; the accumulators are only
//    rescaled when a row max grows by more than 2^8 (exact: P and the row sum share the
//    reference max); P is formed against the current reference while the tile max is found
//    and formed again only when the tile rescales. The row max over the two half-waves is one
//    permlane swap (no LDS), the row sum adds the bf16-rounded P with dot2 instructions.
//  * Causal mask only on the tiles that cross the diagonal (a separate loop, so full tiles run
//    no mask code); keys past the last visible key of the workgroup reuse a valid slot and are
//    masked, so no load leaves the request's slots.
//  * Pool addressing: a per-kv-head base pointer (uniform, in SGPRs) plus a 32-bit byte offset
//    slot * row_bytes (24-bit multiply) when the pool fits (slots * row_bytes <= 2^32, e.g. the
//    2,097,152-slot, 8-head pool of exactly 4 GiB); 64-bit arithmetic otherwise.
//  * Workgroup order is XCD-aware: consecutive workgroup ids go to different XCDs, so the
//    linear id is remapped so that all tiles of one (request, kv head) run on one XCD and
//    share its L2 for the gathered K/V; the longest (last) tiles start first.
#pragma once

#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

namespace {

constexpr int kExtBM = 256;
constexpr int kExtBN = 64;
constexpr int kExtWaves = 8;
constexpr int kExtThreads = 64 * kExtWaves;
constexpr int kXcds = 8;

// Wave priority (s_setprio) over the MFMA blocks of the waves that run each tile whole (waves
// 0-3, the lead group below): when their MFMAs and the other wave of the SIMD (lag group) both
// have an instruction ready, the MFMA goes first, so the matrix pipe does not wait behind the
// lag wave's softmax. Same bits; +1.0-1.6% on the long, mixed and shared-prefix EXTEND steps.
// Raising the lag group's MFMAs above the lead group's measured -3.7%; both at 1, or lead at
// 2 over lag at 1, measured within 0.5% of this.
// FP8 pools: the lead waves widen their share of the next tile between their softmax and their
// P V (rather than after it), so the widened LDS writes land under their own P V MFMAs instead
// of in front of the next iteration's barrier. Same bits; +0.6 to +1.2% on the FP8 EXTEND.
#ifndef RAX_F8_LEAD_EARLY
#define RAX_F8_LEAD_EARLY 1
#endif
#ifndef RAX_EXT_PRIO
#define RAX_EXT_PRIO 1
#endif
#ifndef RAX_PRIO_LEAD
#define RAX_PRIO_LEAD 1
#endif
#ifndef RAX_PRIO_LAG
#define RAX_PRIO_LAG 0
#endif
#if RAX_EXT_PRIO
#define RAX_PRIO_MFMA(PR) __builtin_amdgcn_s_setprio(PR)
#define RAX_PRIO_OTHER() __builtin_amdgcn_s_setprio(0)
#else
#define RAX_PRIO_MFMA(PR)
#define RAX_PRIO_OTHER()
#endif

// In units of 2^kLazyLog2, how far a row max may rise before the accumulators are rescaled.
constexpr float kLazyLog2 = 8.f;

// Row sum of the probabilities: the bf16-rounded P that P V uses, two per v_dot2c_f32_bf16
// against (1, 1), so the normaliser sums exactly the weights applied to V.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_bf16x2(uint32_t pk, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one, acc, false);
}

// LDS swizzles of 16-byte units within a 256-byte row (valid for 32- or 64-bank LDS).
//  K: unit ^ (key & 15): the 16 consecutive rows that one 16-lane phase of an MFMA operand
//     read touches land on 16 distinct units.
//  V: bit 3 of the unit is toggled by bit 1 (the head_dim half a 16-lane group reads), then
//     ^ 2 (key & 3): the four rows of one transposed read (keys 4n .. 4n+3, two units each)
//     land on eight distinct units, and the two 16-lane groups of a half-wave on the other
//     eight.
__device__ __forceinline__ int swz_k(int key, int unit) { return unit ^ (key & 15); }
__device__ __forceinline__ int swz_v(int key, int unit) {
    return (unit ^ (((unit >> 1) & 1) << 3)) ^ (2 * (key & 3));
}
// Logical 16-byte unit stored at physical unit p of V row `key` (inverse of swz_v).
__device__ __forceinline__ int unswz_v(int key, int p) {
    const int t = p ^ (2 * (key & 3));
    return t ^ (((t >> 1) & 1) << 3);
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

// One 16-byte-per-lane HBM -> LDS copy: lane l's 16 bytes land at lds_wave_dst + 16 l
// (gfx950 global_load_lds_dwordx4; the destination is wave-uniform).
__device__ __forceinline__ void lds_dma16(const char* src, void* lds_wave_dst) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_wave_dst, 16, 0, 0);
}

// The same 16-byte-per-lane copy through a buffer resource (buffer_load_dwordx4 ... lds), for
// pools addressed with 32-bit byte offsets. The wait-count bookkeeping of the compiler treats
// the global (FLAT-encoded) form as possibly touching LDS through a flat address and, while one
// is in flight, rounds every LDS and vector-load wait down to zero; the buffer form is a plain
// vector-memory operation, so waits on LDS reads and on slot loads stay exact.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pool_rsrc(const char* base) {
    // raw buffer (stride 0), byte range 2^32 - 1 (offsets are below 2^32 by construction),
    // data format word of gfx9 untyped buffers
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)0xFFFFFFFF, 0x00020000);
}
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_wave_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_dst, 16,
                                             off, 0, 0, 0);
}

template <bool OFF32>
__device__ __forceinline__ const char* pool_row_ptr(const char* base, int slot, uint32_t row_bytes,
                                                    uint32_t off) {
    if constexpr (OFF32) {
        return base + (__umul24((uint32_t)slot, row_bytes) + off);
    } else {
        return base + ((uint64_t)(uint32_t)slot * row_bytes + off);
    }
}

// Slot of key position pos (wave-uniform): the table entry itself, or with a page table the
// page's first slot plus the position within the page.
template <bool PG>
__device__ __forceinline__ int slot_at(const int32_t* row, int pos, int page_shift) {
    if constexpr (PG) return (row[pos >> page_shift] << page_shift) | (pos & ((1 << page_shift) - 1));
    else return row[pos];
}

// Byte offset of row `idx` (a pool slot, or a new row of the ragged suffix): a 24-bit multiply
// when both the pool and the new rows fit 32-bit offsets (OFF32), 64-bit otherwise.
template <bool OFF32>
__device__ __forceinline__ int64_t row_off(int idx, uint32_t row_bytes) {
    if constexpr (OFF32) return (int64_t)__umul24((uint32_t)idx, row_bytes);
    else return (int64_t)(uint32_t)idx * row_bytes;
}


// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
#define RAX_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | (((N) >> 4) << 14)) | 0x0F70)
// Workgroup barrier that the compiler may not move memory accesses across. Copies into LDS
// are ordered by the explicit vmcnt wait before it, reads by the operand waits of the MFMAs.
#define RAX_BARRIER() asm volatile("s_barrier" ::: "memory")
// Barrier after which other waves read this wave's LDS writes: the wait for them and the
// barrier are one statement, so no write can be scheduled between the two.
#define RAX_WRITES_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// PG: the table is a page table (page size 2^page_shift): position j lives at slot
// table[row, j >> page_shift] << page_shift | (j & (2^page_shift - 1)).
// SPL: the key range of each row tile is split over nsplit workgroups, which write partial
// outputs (fp32, normalised) and their log2-sum-exps to o_part / lse_part for
// extend_merge_kernel.
template <int DH, int G, bool OFF32, bool KV8, bool RAG, bool PG, bool SPL>
__global__ __launch_bounds__(kExtThreads, 1) void extend_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const char* __restrict__ k_pool,
    const char* __restrict__ v_pool, const char* __restrict__ k_new, const char* __restrict__ v_new,
    const int32_t* __restrict__ store_loc, const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ extend_start_loc,
    int64_t total_tokens, int32_t max_extend_len, int32_t max_seq_len, int32_t Hq, int32_t Hkv,
    int32_t batch, int32_t tiles, float scale_log2, float out_scale, int32_t page_shift,
    int32_t spread_shift, int32_t nsplit, float* __restrict__ o_part, float* __restrict__ lse_part) {
    // head_dim of Q, O and the pool rows. The LDS tiles keep 128-wide rows either way: with
    // head_dim 64 only logical units 0-7 of a row are used (score steps 0-3, P V blocks 0-1)
    // and the copy lanes of units 8-15 fetch a copy of units 0-7, so no copy leaves its row.
    constexpr int D = DH;
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");

    // Score of a masked key. A split's tiles can hold no visible key for some rows (all past
    // the row's diagonal): with a finite mask value those rows keep a finite running max and
    // finite sums, and a log2-sum-exp near -2^100 * scale that gives their partial weight 0
    // in the merge, where -inf would turn the online softmax into NaN. A power of two keeps
    // the scaled value exact: the running max (a rounded product) and the exponent argument
    // (a fused multiply-add with the unrounded product) then cancel to exactly 0 instead of
    // leaving a rounding residual of order 1e21.
    constexpr float kMasked = SPL ? -0x1p100f : -INFINITY;
    // G = 0: the group size is read at run time (Hq / Hkv) and each workgroup takes
    // floor(256 / G) tokens; the rows past BQ * G of the tile are idle (computed, never stored).
    const int Gv = G > 0 ? G : Hq / Hkv;
    const int BQ = kExtBM / Gv;  // tokens per workgroup
    constexpr int EB = KV8 ? 1 : 2;  // bytes per pool element
    static_assert(!(KV8 && RAG), "ragged suffix rows are bf16, as the pools");

    // Three K/V tile buffers, row-major [key][16 units of 8 bf16], swizzled. Separate LDS
    // objects, each named statically below.
    __shared__ uint4 kb0[kExtBN * 16], kb1[kExtBN * 16], kb2[kExtBN * 16];
    __shared__ uint4 vb0[kExtBN * 16], vb1[kExtBN * 16], vb2[kExtBN * 16];
    __shared__ uint4 kb3[kExtBN * 16], vb3[kExtBN * 16];  // fourth buffer (ping-pong, below)
    // FP8 pools: two staging buffers of raw E4M3 tiles, [key][8 units of 16 bytes] (with the
    // four bf16 buffers, 160 KB of LDS).
    constexpr int SU = KV8 ? kExtBN * 8 : 1;
    __shared__ uint4 sk0[SU], sk1[SU], sv0[SU], sv1[SU];

    // ---- workgroup -> (pair = b * Hkv + g, tile), XCD-aware. Consecutive workgroup ids go
    // to different XCDs; XCD x takes every tile of pairs x, x + 8, ... of the first multiple of
    // 8 pairs (one L2 per pair), longest tile first. The rem = pairs % 8 pairs past that
    // multiple (all of them when there are fewer than 8) are spread: each takes
    // 2^spread_shift XCDs (the power of two at most 8 / rem), which share its tiles round
    // robin, so no XCD stays idle for want of a pair.
    const int pairs = batch * Hkv;
    // SPL: split sp of the key range; the grid is nsplit copies of the unsplit one, each a
    // multiple of 8 workgroups long, so a workgroup keeps its XCD.
    int bid = blockIdx.x, sp = 0;
    if constexpr (SPL) {
        const int per_split = gridDim.x / nsplit;
        sp = bid / per_split;
        bid -= sp * per_split;
    }
    const int xcd = bid % kXcds;
    const int k = bid / kXcds;
    const int full = pairs & ~(kXcds - 1);
    const int rounds = (pairs / kXcds) * tiles;  // per-XCD slots of the full groups of 8
    int pair, jt;
    if (k < rounds) {
        pair = xcd + kXcds * (k / tiles);
        jt = k % tiles;
    } else {
        pair = full + (xcd >> spread_shift);
        jt = ((k - rounds) << spread_shift) + (xcd & ((1 << spread_shift) - 1));
        if (pair >= pairs || jt >= tiles) return;
    }
    const int tq = tiles - 1 - jt;
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
    const uint32_t row_bytes = (uint32_t)Hkv * D * EB;
    const char* kbase = k_pool + (int64_t)g * D * EB;
    const char* vbase = v_pool + (int64_t)g * D * EB;
    const __amdgpu_buffer_rsrc_t krsrc = pool_rsrc(kbase);  // used by the 32-bit-offset copies
    const __amdgpu_buffer_rsrc_t vrsrc = pool_rsrc(vbase);
    // Ragged suffix: key position j >= p is new row s0 + j - p of k_new / v_new ([tokens, Hkv,
    // D], the same row size as the pool), the prefix comes from the pool.
    const char* knbase = RAG ? k_new + (int64_t)g * D * EB : nullptr;
    const char* vnbase = RAG ? v_new + (int64_t)g * D * EB : nullptr;
    const __amdgpu_buffer_rsrc_t knrsrc = pool_rsrc(RAG ? knbase : kbase);
    const __amdgpu_buffer_rsrc_t vnrsrc = pool_rsrc(RAG ? vnbase : vbase);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;  // query row within the wave (MFMA N index)
    const int h2 = lane >> 5;   // k-group of the MFMA operands

    // ---- this lane's query row
    const int r = 32 * wave + col;
    const int t = t0 + r / Gv;
    const int hl = r % Gv;
    const bool row_ok = (G > 0 || r < BQ * Gv) && t < e;  // with G > 0, BQ * G = 256 rows
    const int t_ld = row_ok ? t : e - 1;
    const int64_t qo_row = ((int64_t)(s0 + t_ld) * Hq + (int64_t)g * Gv + hl) * D;
    bf16x8 qop[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = as_bf16x8(*(const uint4*)(q + qo_row + 16 * s + 8 * h2));

    // ---- HBM -> LDS copies. Copy instruction i (0, 1) of wave w fills tile rows
    // R = 8 w + 4 i + lane / 16, physical unit lane % 16 each; the lane fetches the logical
    // unit the swizzle stores there: R & 15 = 8 (w & 1) + 4 i + prow, R & 3 = prow.
    const int prow = lane >> 4;
    const int punit = lane & 15;
    const uint32_t k_src0 = 16u * (uint32_t)((punit ^ (8 * (wave & 1) + prow)) & (D / 8 - 1));
    const uint32_t k_src1 = 16u * (uint32_t)((punit ^ (8 * (wave & 1) + 4 + prow)) & (D / 8 - 1));
    const uint32_t v_src = 16u * (uint32_t)(unswz_v(prow, punit) & (D / 8 - 1));
    // SPL: this workgroup takes key tiles [it_lo, it_lo + ntiles) of the row tile's, split sp
    // of nsplit near-equal blocks (possibly none); kofs is the first key's position.
    int ntiles = (kend + kExtBN - 1) / kExtBN;
    int it_lo = 0;
    if constexpr (SPL) {
        const int all = ntiles;
        it_lo = (int)((int64_t)all * sp / nsplit);
        ntiles = (int)((int64_t)all * (sp + 1) / nsplit) - it_lo;
    }
    const int kofs = it_lo * kExtBN;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // bf16 pools: the slot numbers of the two rows a lane copies (tile rows 8 w + prow and
    // 8 w + 4 + prow) come through per-lane vector loads, one tile before their copy. Scalar
    // loads would share the LDS counter (lgkmcnt) and, being unordered, turn every LDS operand
    // wait of the next tile into a wait for all of them; vector loads count on vmcnt, in order
    // with the copies, so the explicit copy waits below account for them. Tile T's slots are
    // held in register set T % 2 (S0, S1).
#define RAX_VSLOTS(TILE, S0, S1)                                                            \
    {                                                                                       \
        const int p0_ = min(kofs + (TILE) * kExtBN + 8 * wave + prow, kend - 1);           \
        const int p1_ = min(kofs + (TILE) * kExtBN + 8 * wave + 4 + prow, kend - 1);       \
        S0 = slot_at<PG>(row, p0_, page_shift);                                            \
        S1 = slot_at<PG>(row, p1_, page_shift);                                            \
    }
    // Ragged suffix with 32-bit offsets: a copied row comes from the pool (prefix position) or
    // from the new rows (suffix position), each through its own buffer resource. The two forms
    // are the two arms of a per-lane branch, run under complementary lane masks (both arms only
    // on the tile that straddles the prefix end), so a tile still issues at least the 4 copies
    // the explicit waits count. As the compiler must assume either arm may be skipped, its own
    // waits for the slot registers count no copy: the offsets of both rows are therefore formed
    // before any of the tile's copies is issued (and, in the loop, before the next slot loads).
#define RAX_RADDR(TILE, S0, S1, N0, N1, O0, O1)                                             \
    {                                                                                       \
        const int ps0_ = min(kofs + (TILE) * kExtBN + 8 * wave + prow, kend - 1);          \
        const int ps1_ = min(kofs + (TILE) * kExtBN + 8 * wave + 4 + prow, kend - 1);      \
        N0 = ps0_ >= p;                                                                     \
        N1 = ps1_ >= p;                                                                     \
        O0 = __umul24((uint32_t)(N0 ? s0 + ps0_ - p : (S0)), row_bytes);                   \
        O1 = __umul24((uint32_t)(N1 ? s0 + ps1_ - p : (S1)), row_bytes);                   \
    }
#define RAX_RISSUE(KB, VB, N0, N1, O0, O1)                                                  \
    {                                                                                       \
        char* kd_ = (char*)(KB) + (8 * wave_u) * 256;                                       \
        char* vd_ = (char*)(VB) + (8 * wave_u) * 256;                                       \
        /* the empty statement in one arm keeps the compiler from merging the arms into */  \
        /* one copy with a per-lane resource (a loop over the distinct resources) */         \
        if (N0) {                                                                           \
            lds_dma16_buf(knrsrc, (O0) + k_src0, kd_);                                      \
            lds_dma16_buf(vnrsrc, (O0) + v_src, vd_);                                       \
            asm volatile("" ::: "memory");                                                  \
        } else {                                                                            \
            lds_dma16_buf(krsrc, (O0) + k_src0, kd_);                                       \
            lds_dma16_buf(vrsrc, (O0) + v_src, vd_);                                        \
        }                                                                                   \
        if (N1) {                                                                           \
            lds_dma16_buf(knrsrc, (O1) + k_src1, kd_ + 1024);                               \
            lds_dma16_buf(vnrsrc, (O1) + v_src, vd_ + 1024);                                \
            asm volatile("" ::: "memory");                                                  \
        } else {                                                                            \
            lds_dma16_buf(krsrc, (O1) + k_src1, kd_ + 1024);                                \
            lds_dma16_buf(vrsrc, (O1) + v_src, vd_ + 1024);                                 \
        }                                                                                   \
    }
#define RAX_VCOPY(KB, VB, TILE, S0, S1)                                                     \
    {                                                                                       \
        char* kd_ = (char*)(KB) + (8 * wave_u) * 256;                                       \
        char* vd_ = (char*)(VB) + (8 * wave_u) * 256;                                       \
        if constexpr (!RAG && OFF32) {                                                      \
            const uint32_t o0_ = __umul24((uint32_t)(S0), row_bytes);                       \
            const uint32_t o1_ = __umul24((uint32_t)(S1), row_bytes);                       \
            lds_dma16_buf(krsrc, o0_ + k_src0, kd_);                                        \
            lds_dma16_buf(krsrc, o1_ + k_src1, kd_ + 1024);                                 \
            lds_dma16_buf(vrsrc, o0_ + v_src, vd_);                                         \
            lds_dma16_buf(vrsrc, o1_ + v_src, vd_ + 1024);                                  \
        } else if constexpr (!RAG) {                                                        \
            lds_dma16(pool_row_ptr<OFF32>(kbase, S0, row_bytes, k_src0), kd_);              \
            lds_dma16(pool_row_ptr<OFF32>(kbase, S1, row_bytes, k_src1), kd_ + 1024);       \
            lds_dma16(pool_row_ptr<OFF32>(vbase, S0, row_bytes, v_src), vd_);               \
            lds_dma16(pool_row_ptr<OFF32>(vbase, S1, row_bytes, v_src), vd_ + 1024);        \
        } else {                                                                            \
            const int ps0_ = min(kofs + (TILE) * kExtBN + 8 * wave + prow, kend - 1);      \
            const int ps1_ = min(kofs + (TILE) * kExtBN + 8 * wave + 4 + prow, kend - 1);  \
            const bool n0_ = ps0_ >= p, n1_ = ps1_ >= p;                                    \
            const int64_t r0_ = row_off<OFF32>(n0_ ? s0 + ps0_ - p : S0, row_bytes);        \
            const int64_t r1_ = row_off<OFF32>(n1_ ? s0 + ps1_ - p : S1, row_bytes);        \
            lds_dma16((n0_ ? knbase : kbase) + (r0_ + k_src0), kd_);                        \
            lds_dma16((n1_ ? knbase : kbase) + (r1_ + k_src1), kd_ + 1024);                 \
            lds_dma16((n0_ ? vnbase : vbase) + (r0_ + v_src), vd_);                         \
            lds_dma16((n1_ ? vnbase : vbase) + (r1_ + v_src), vd_ + 1024);                  \
        }                                                                                   \
    }
    // FP8 pools: a 64-key tile is 8 KB per operand, so one copy instruction per wave moves
    // its eight rows: lane l fetches 16 bytes at offset 16 (l % 8) of row 8 w + l / 8 into
    // staging unit 64 w + l. The lane's slot comes through a per-lane vector load (tile T's in
    // register set T % 2), as for bf16 pools. Per wave and tile: 1 slot load, 2 copies. With
    // head_dim 64 a row is 4 units: lanes of units 4-7 fetch a copy of units 0-3, whose
    // widening lands in logical units 8-15 of the bf16 row, which head_dim 64 does not read.
    const int q8 = lane >> 3;
    const uint32_t src8 = 16u * (uint32_t)(lane & 7 & (D / 16 - 1));
#define RAX_VSLOT8(TILE, S)                                                                 \
    {                                                                                       \
        S = slot_at<PG>(row, min(kofs + (TILE) * kExtBN + 8 * wave + q8, kend - 1), page_shift); \
    }
#define RAX_COPY8(SK, SV, S)                                                                \
    {                                                                                       \
        if constexpr (OFF32) {                                                              \
            const uint32_t o_ = __umul24((uint32_t)(S), row_bytes) + src8;                  \
            lds_dma16_buf(krsrc, o_, (char*)(SK) + wave_u * 1024);                          \
            lds_dma16_buf(vrsrc, o_, (char*)(SV) + wave_u * 1024);                          \
        } else {                                                                            \
            lds_dma16(pool_row_ptr<OFF32>(kbase, S, row_bytes, src8), (char*)(SK) + wave_u * 1024); \
            lds_dma16(pool_row_ptr<OFF32>(vbase, S, row_bytes, src8), (char*)(SV) + wave_u * 1024); \
        }                                                                                   \
    }
    // Each lane widens the staging unit it copied (16 E4M3 values = head_dim 16 u .. 16 u + 15
    // of key 8 w + l / 8) into logical units 2 u and 2 u + 1 of the swizzled bf16 tile. Only
    // the lane's own copy must have landed (vmcnt); the barrier before the tile's use makes
    // the bf16 tile visible to the other waves.
    const int ckey = 8 * wave + q8;
    const int cu2 = 2 * (lane & 7);
#define RAX_CONVERT8(SK, SV, KB, VB)                                                        \
    {                                                                                       \
        const uint4 k8_ = (SK)[64 * wave + lane];                                           \
        const uint4 v8_ = (SV)[64 * wave + lane];                                           \
        (KB)[ckey * 16 + swz_k(ckey, cu2)] = widen8(make_uint2(k8_.x, k8_.y));              \
        (KB)[ckey * 16 + swz_k(ckey, cu2 + 1)] = widen8(make_uint2(k8_.z, k8_.w));          \
        (VB)[ckey * 16 + swz_v(ckey, cu2)] = widen8(make_uint2(v8_.x, v8_.y));              \
        (VB)[ckey * 16 + swz_v(ckey, cu2 + 1)] = widen8(make_uint2(v8_.z, v8_.w));          \
    }

    // ---- per-lane constants of the transposed V reads: 16-lane group gi holds head_dim half
    // dh = gi & 1 and k-group h2; lane i16 = 4 jr + cc reads key offset jr and head_dim
    // 4 cc .. 4 cc + 3 of that half.
    const int i16 = lane & 15;
    const int dh = (lane >> 4) & 1;
    const int jr = i16 >> 2;
    const int cc = i16 & 3;

    float m = -INFINITY;
    float lsum = 0.f, lsum2 = 0.f;  // row sum in two interleaved parts (shorter dependency chain)
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    const int last_q = p + t;        // last key position this row may see
    const int diag_from = p + t0;    // a tile whose last key exceeds this needs the mask

    // Per tile: scores (QK), (mask,) softmax (SM), P V (PV). An iteration waits for its tile's
    // copies, passes the barrier, computes, then starts the copy of tile IT+2 into a buffer
    // every wave finished with before the barrier. Issuing the copy after this tile's LDS reads
    // keeps the copies in flight where the reads happen to buffers the compiler can tell apart,
    // so it adds no waits of its own. The only vector-memory operations are the copies (4 per
    // tile), issued two tiles ahead: when tile IT is needed the younger ones are the copies of
    // IT+1, so wait until at most 4 are outstanding (0 at the last tile of the masked tail,
    // whose copies stop at the last tile). The unmasked steady loop copies unconditionally, also
    // past the last tile (positions clamp to the last key; the buffers are not read again), and
    // runs until fewer than four full tiles remain; the copies still in flight after the loops
    // are drained before the workgroup ends.
    f32x16 st[2];   // scores of the tile being processed
    uint4 pf[4];    // its probabilities (bf16), the B operand of P V
    // The two 32-key halves of the tile are independent accumulation chains; each K-dim step
    // reads both halves' operands and issues both MFMAs, so one pair of LDS reads feeds 64
    // MFMA cycles and no operand waits in registers for the other chain.
#define RAX_QKP(KB, PR)                                                                     \
    {                                                                                       \
        RAX_PRIO_MFMA(PR);                                                                  \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                    \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) st[mb][i] = 0.f;                     \
        uint4 ka0_ = (KB)[col * 16 + swz_k(col, h2)];                                       \
        uint4 ka1_ = (KB)[(32 + col) * 16 + swz_k(32 + col, h2)];                           \
        _Pragma("unroll") for (int s = 0; s < D / 16; ++s) {                                \
            uint4 kb0_ = ka0_, kb1_ = ka1_;                                                 \
            if (s + 1 < D / 16) {     /* the next step's operands, read one step ahead */   \
                kb0_ = (KB)[col * 16 + swz_k(col, 2 * (s + 1) + h2)];                       \
                kb1_ = (KB)[(32 + col) * 16 + swz_k(32 + col, 2 * (s + 1) + h2)];           \
            }                                                                               \
            st[0] = mfma32x32x16(as_bf16x8(ka0_), qop[s], st[0]);                           \
            st[1] = mfma32x32x16(as_bf16x8(ka1_), qop[s], st[1]);                           \
            ka0_ = kb0_;                                                                    \
            ka1_ = kb1_;                                                                    \
        }                                                                                   \
        /* keep that order: 2 reads, then per step 2 reads of the next step and 2 MFMAs */  \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                  \
        _Pragma("unroll") for (int s = 0; s < D / 16 - 1; ++s) {                            \
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                              \
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                              \
        }                                                                                   \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                  \
        RAX_PRIO_OTHER();                                                                   \
    }
    // P = 2^(scale_log2 * s - m) rounded to bf16 into pf (the B operand of P V), added two at a
    // time into the row sums lsum / lsum2.
#define RAX_PEXP()                                                                          \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                      \
        float pv[8];                                                                        \
        _Pragma("unroll") for (int j = 0; j < 8; ++j)                                       \
            pv[j] = fast_exp2(fmaf(st[kk >> 1][8 * (kk & 1) + j], scale_log2, -m));         \
        pf[kk].x = pack_bf16x2(pv[0], pv[1]);                                               \
        pf[kk].y = pack_bf16x2(pv[2], pv[3]);                                               \
        pf[kk].z = pack_bf16x2(pv[4], pv[5]);                                               \
        pf[kk].w = pack_bf16x2(pv[6], pv[7]);                                               \
        lsum = add_bf16x2(pf[kk].x, lsum);                                                  \
        lsum2 = add_bf16x2(pf[kk].y, lsum2);                                                \
        lsum = add_bf16x2(pf[kk].z, lsum);                                                  \
        lsum2 = add_bf16x2(pf[kk].w, lsum2);                                                \
    }
#define RAX_SM(IT, MASKABLE)                                                                \
    {                                                                                       \
        if (MASKABLE && __builtin_amdgcn_readfirstlane(kofs + (IT) * kExtBN + kExtBN - 1 > diag_from)) { \
            const int j0_ = kofs + (IT) * kExtBN;                                           \
            _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                \
            _Pragma("unroll") for (int jj = 0; jj < 4; ++jj)                                \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                 \
                if (j0_ + 32 * mb + 8 * jj + 4 * h2 + i > last_q) st[mb][4 * jj + i] = kMasked; \
            }                                                                               \
        }                                                                                   \
        /* P is formed against the current reference maximum m while the tile's maximum is  */ \
        /* found, so the exponentials do not wait for the max chain; that P is the result     */ \
        /* unless the tile raises some row's maximum by more than 2^kLazyLog2 (always on the  */ \
        /* first tile, m = -inf), when the sums are restored, rescaled and P is formed again. */ \
        const float l0_ = lsum, l1_ = lsum2;                                                \
        float mx = -INFINITY;                                                               \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                    \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[mb][i]);           \
        RAX_PEXP()                                                                          \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk)                                    \
            asm volatile("" : "+v"(pf[kk].x), "+v"(pf[kk].y), "+v"(pf[kk].z), "+v"(pf[kk].w)); \
        asm volatile("" : "+v"(lsum), "+v"(lsum2));                                         \
        mx = max_pair32(mx) * scale_log2;                                                   \
        if (__any(mx > m + kLazyLog2)) {                                                    \
            const float m_new = fmaxf(m, mx);                                               \
            const float alpha = fast_exp2(m - m_new);                                       \
            m = m_new;                                                                      \
            lsum = l0_ * alpha;                                                             \
            lsum2 = l1_ * alpha;                                                            \
            _Pragma("unroll") for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;         \
            RAX_PEXP()                                                                      \
        }                                                                                   \
    }
    // V^T operand of step (dt, kk): two transposed reads of keys 16 kk + 4 h2 + jr (+ 8).
#define RAX_VREAD(VBB, DT, KK)                                                              \
    ({                                                                                      \
        const int unit_ = 4 * (DT) + 2 * dh + (cc >> 1);                                    \
        const int key0_ = 16 * (KK) + 4 * h2 + jr;                                          \
        const int key1_ = key0_ + 8;                                                        \
        const uint2 h0_ = ds_read_tr16_b64((VBB) + key0_ * 256 + swz_v(key0_, unit_) * 16 + 8 * (cc & 1)); \
        const uint2 h1_ = ds_read_tr16_b64((VBB) + key1_ * 256 + swz_v(key1_, unit_) * 16 + 8 * (cc & 1)); \
        make_uint4(h0_.x, h0_.y, h1_.x, h1_.y);                                             \
    })
    // 16 steps (kk, dt), key step major, each operand read two steps ahead of its MFMA. Each
    // accumulator still adds its key steps in order 0..3; consecutive MFMAs share their P
    // operand, which measured +1.3% on the long-context step (power-limited) and no change on
    // the shorter ones.
#define RAX_PVP(VB, PR)                                                                     \
    {                                                                                       \
        RAX_PRIO_MFMA(PR);                                                                  \
        const char* vbb = (const char*)(VB);                                                \
        uint4 va_ = RAX_VREAD(vbb, 0, 0);                                                   \
        uint4 vb_ = RAX_VREAD(vbb, 1 % (D / 32), 1 / (D / 32));                             \
        _Pragma("unroll") for (int st_ = 0; st_ < D / 8; ++st_) {                           \
            const int dt = st_ % (D / 32), kk = st_ / (D / 32);                             \
            uint4 vc_ = vb_;                                                                \
            if (st_ + 2 < D / 8) vc_ = RAX_VREAD(vbb, (st_ + 2) % (D / 32), (st_ + 2) / (D / 32)); \
            acc[dt] = mfma32x32x16(as_bf16x8(va_), as_bf16x8(pf[kk]), acc[dt]);             \
            va_ = vb_;                                                                      \
            vb_ = vc_;                                                                      \
        }                                                                                   \
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                  \
        _Pragma("unroll") for (int st_ = 0; st_ < D / 8 - 2; ++st_) {                       \
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                              \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
        }                                                                                   \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                  \
        RAX_PRIO_OTHER();                                                                   \
    }
#define RAX_QK(KB) RAX_QKP(KB, RAX_PRIO_LEAD)
#define RAX_PV(VB) RAX_PVP(VB, RAX_PRIO_LEAD)
#define RAX_COMPUTE(IT, KB, VB, MASKABLE) { RAX_QK(KB) RAX_SM(IT, MASKABLE) RAX_PV(VB) }
    // Ping-pong (4 LDS buffers): waves w and w + 4 share a SIMD. Waves 0-3 run tile IT whole
    // (scores, softmax, P V); waves 4-7 run the softmax and P V of tile IT-1 and then the
    // scores of tile IT, so that on each SIMD one wave's MFMAs meet the other's softmax. Tile
    // IT-1's V stays readable during iteration IT: the copy started in iteration IT goes to
    // the buffer of tile IT-2.
#define RAX_PCOMPUTE(LAG, IT, KB, VB, VP, MASKABLE, STEADY)                                 \
    {                                                                                       \
        if (LAG) {                                                                          \
            if (!STEADY && (IT) == 0) {                                                     \
            } else {                                                                        \
                RAX_SM((IT) - 1, MASKABLE) RAX_PVP(VP, RAX_PRIO_LAG)                        \
            }                                                                               \
            RAX_QKP(KB, RAX_PRIO_LAG)                                                       \
        } else {                                                                            \
            RAX_COMPUTE(IT, KB, VB, MASKABLE)                                               \
        }                                                                                   \
    }
    // Vector-memory operations per wave and tile: at the end of iteration IT, the 2 slot loads
    // of tile IT+3 (into set (IT+3) % 2), then the 4 copies of tile IT+2 (set (IT+2) % 2). At the
    // start of iteration IT the copies of tile IT are needed; younger are the slot loads of tile
    // IT+2 and the copies of tile IT+1 (issued at the end of IT-1, when those tiles exist, and
    // always in the steady loop): wait until at most 6, 4 or 0 operations are outstanding.
#define RAX_PTILE(LAG, IT, KB, VB, VP, KN, VN, SU0, SU1, SL0, SL1, MASKABLE, STEADY)        \
    {                                                                                       \
        if (STEADY || (IT) + 2 < ntiles) {                                                  \
            RAX_WAIT_VMCNT(6);                                                              \
        } else if ((IT) + 1 < ntiles) {                                                     \
            RAX_WAIT_VMCNT(4);                                                              \
        } else {                                                                            \
            RAX_WAIT_VMCNT(0);                                                              \
        }                                                                                   \
        RAX_BARRIER();                                                                      \
        RAX_PCOMPUTE(LAG, IT, KB, VB, VP, MASKABLE, STEADY)                                 \
        if constexpr (RAG && OFF32) {                                                       \
            bool rn0_ = false, rn1_ = false;                                                \
            uint32_t ro0_ = 0, ro1_ = 0;                                                    \
            if (STEADY || (IT) + 2 < ntiles) {                                              \
                RAX_RADDR((IT) + 2, SU0, SU1, rn0_, rn1_, ro0_, ro1_)                       \
                asm volatile("" ::"v"(ro0_), "v"(ro1_) : "memory");                        \
            }                                                                               \
            if (STEADY || (IT) + 3 < ntiles) RAX_VSLOTS((IT) + 3, SL0, SL1)                 \
            if (STEADY || (IT) + 2 < ntiles) RAX_RISSUE(KN, VN, rn0_, rn1_, ro0_, ro1_)     \
        } else {                                                                            \
            if (STEADY || (IT) + 3 < ntiles) RAX_VSLOTS((IT) + 3, SL0, SL1)                 \
            if (STEADY || (IT) + 2 < ntiles) RAX_VCOPY(KN, VN, (IT) + 2, SU0, SU1)          \
        }                                                                                   \
    }
    // FP8 pools: tile T is staged (E4M3) in buffer T % 2 and widened into bf16 buffer T % 4;
    // its slot is held in register set T % 2. Iteration IT: barrier (every wave's widening of
    // tile IT has landed, every wave is done with iteration IT-1, whose widening read staging
    // IT % 2); copy tile IT+2 into staging IT % 2 (slot set SS); compute as above; wait for
    // this wave's copies of tile IT+1 and widen them from staging (SC, SVC) into (KN, VN), free
    // since tile IT-3; then load the slot of tile IT+4 into set SS (the copy has taken its
    // address already). When tile IT+1 is widened, the operations younger than its copies are
    // the slot load of tile IT+3 (iteration IT-1) and the copies of tile IT+2 (this iteration),
    // when those tiles exist (always in the steady loop): wait until at most 3, 2 or 0 are
    // outstanding.
#define RAX_WIDEN8(IT, SC, SVC, KN, VN, SS, STEADY)                                         \
    {                                                                                       \
        if (STEADY || (IT) + 1 < ntiles) {                                                  \
            if (STEADY || (IT) + 3 < ntiles) {                                              \
                RAX_WAIT_VMCNT(3);                                                          \
            } else if ((IT) + 2 < ntiles) {                                                 \
                RAX_WAIT_VMCNT(2);                                                          \
            } else {                                                                        \
                RAX_WAIT_VMCNT(0);                                                          \
            }                                                                               \
            RAX_CONVERT8(SC, SVC, KN, VN)                                                   \
        }                                                                                   \
        if (STEADY || (IT) + 4 < ntiles) RAX_VSLOT8((IT) + 4, SS)                           \
    }
    // Waves 4-7 widen between their P V and their scores, so that per iteration each wave
    // group alternates MFMA and VALU/LDS blocks in the opposite order to the other group
    // (+1 to +3% over widening at the end of the iteration in both groups); waves 0-3 widen
    // between their softmax and their P V (RAX_F8_LEAD_EARLY). Widening first thing in the
    // iteration (waves 4-7) measured the same.
#define RAX_PTILE8(LAG, IT, KB, VB, VP, SC, SVC, SCP, SVCP, KN, VN, SS, MASKABLE, STEADY)    \
    {                                                                                       \
        RAX_WRITES_BARRIER();                                                               \
        if (STEADY || (IT) + 2 < ntiles) RAX_COPY8(SCP, SVCP, SS)                           \
        if (LAG) {                                                                          \
            if (!STEADY && (IT) == 0) {                                                     \
            } else {                                                                        \
                RAX_SM((IT) - 1, MASKABLE) RAX_PVP(VP, RAX_PRIO_LAG)                        \
            }                                                                               \
            RAX_WIDEN8(IT, SC, SVC, KN, VN, SS, STEADY)                                     \
            /* the staging reads would fill the first LDS-read group of the scores */       \
            __builtin_amdgcn_sched_barrier(0);                                              \
            RAX_QKP(KB, RAX_PRIO_LAG)                                                       \
        } else if (RAX_F8_LEAD_EARLY) {                                                     \
            RAX_QK(KB)                                                                      \
            RAX_SM(IT, MASKABLE)                                                            \
            RAX_WIDEN8(IT, SC, SVC, KN, VN, SS, STEADY)                                     \
            __builtin_amdgcn_sched_barrier(0);                                              \
            RAX_PV(VB)                                                                      \
        } else {                                                                            \
            RAX_COMPUTE(IT, KB, VB, MASKABLE)                                               \
            RAX_WIDEN8(IT, SC, SVC, KN, VN, SS, STEADY)                                     \
        }                                                                                   \
    }


    // tiles with every key <= p + t0
    const int n_full = max(0, min(ntiles, (diag_from + 1) / kExtBN - it_lo));
    int it = 0;
    const bool lag = __builtin_amdgcn_readfirstlane(wave) >= 4;
    if constexpr (SPL) {
        if (ntiles == 0) {  // no key of this split: a partial of weight 0 (uniform per workgroup)
            if (row_ok) {
                const int64_t prow_ = (int64_t)sp * total_tokens * Hq * D + qo_row;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        *(float4*)(o_part + prow_ + 32 * dt + 8 * jj + 4 * h2) = make_float4(0.f, 0.f, 0.f, 0.f);
                if (h2 == 0) lse_part[(int64_t)sp * total_tokens * Hq + qo_row / D] = -INFINITY;
            }
            return;
        }
    }
    // waves 4-7 after their loop: softmax and P V of the last tile (inside their branch, so
    // the scores stay dead after the softmax for waves 0-3)
#define RAX_LAG_TAIL()                                                                      \
    {                                                                                       \
        RAX_SM(ntiles - 1, 1)                                                               \
        switch ((ntiles - 1) & 3) {                                                         \
            case 0: RAX_PVP(vb0, RAX_PRIO_LAG) break;                                       \
            case 1: RAX_PVP(vb1, RAX_PRIO_LAG) break;                                       \
            case 2: RAX_PVP(vb2, RAX_PRIO_LAG) break;                                       \
            default: RAX_PVP(vb3, RAX_PRIO_LAG) break;                                      \
        }                                                                                   \
    }
    if constexpr (!KV8) {
        // slots of tiles 0 and 1 (the compiler waits for them before the copies), copies of
        // tiles 0 and 1, then the slots of tile 2 into set 0
        int sl_a0, sl_a1, sl_b0, sl_b1;  // slot register sets 0 (a) and 1 (b)
        RAX_VSLOTS(0, sl_a0, sl_a1)
        if (ntiles > 1) RAX_VSLOTS(1, sl_b0, sl_b1)
        if constexpr (RAG && OFF32) {
            // both tiles' offsets before the first copy (see RAX_RADDR)
            bool n0a, n1a, n0b = false, n1b = false;
            uint32_t o0a, o1a, o0b = 0, o1b = 0;
            RAX_RADDR(0, sl_a0, sl_a1, n0a, n1a, o0a, o1a)
            if (ntiles > 1) RAX_RADDR(1, sl_b0, sl_b1, n0b, n1b, o0b, o1b)
            asm volatile("" ::"v"(o0a), "v"(o1a), "v"(o0b), "v"(o1b) : "memory");
            RAX_RISSUE(kb0, vb0, n0a, n1a, o0a, o1a)
            if (ntiles > 1) RAX_RISSUE(kb1, vb1, n0b, n1b, o0b, o1b)
        } else {
            RAX_VCOPY(kb0, vb0, 0, sl_a0, sl_a1)
            if (ntiles > 1) RAX_VCOPY(kb1, vb1, 1, sl_b0, sl_b1)
        }
        if (ntiles > 2) RAX_VSLOTS(2, sl_a0, sl_a1)
        // Tile T lives in buffer T % 4; iteration T starts the copy of tile T+2 into buffer
        // (T+2) % 4 with slot set (T+2) % 2 and loads the slots of tile T+3 into set (T+3) % 2.
        // The first iteration is peeled (waves 4-7 have no previous tile there); the steady
        // loop starts at an odd tile and is unrolled by four, so buffers and sets are static.
        // One loop nest per wave group (the same barriers in the same order), so that the
        // scores carried across iterations by waves 4-7 cost registers only there.
#define RAX_PLOOPS(LAG)                                                                     \
        RAX_PTILE(LAG, it, kb0, vb0, vb3, kb2, vb2, sl_a0, sl_a1, sl_b0, sl_b1, 1, 0) ++it;  \
        while (it + 4 <= n_full) {                                                          \
            RAX_PTILE(LAG, it, kb1, vb1, vb0, kb3, vb3, sl_b0, sl_b1, sl_a0, sl_a1, 0, 1) ++it; \
            RAX_PTILE(LAG, it, kb2, vb2, vb1, kb0, vb0, sl_a0, sl_a1, sl_b0, sl_b1, 0, 1) ++it; \
            RAX_PTILE(LAG, it, kb3, vb3, vb2, kb1, vb1, sl_b0, sl_b1, sl_a0, sl_a1, 0, 1) ++it; \
            RAX_PTILE(LAG, it, kb0, vb0, vb3, kb2, vb2, sl_a0, sl_a1, sl_b0, sl_b1, 0, 1) ++it; \
        }                                                                                   \
        while (it < ntiles) {                                                               \
            RAX_PTILE(LAG, it, kb1, vb1, vb0, kb3, vb3, sl_b0, sl_b1, sl_a0, sl_a1, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE(LAG, it, kb2, vb2, vb1, kb0, vb0, sl_a0, sl_a1, sl_b0, sl_b1, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE(LAG, it, kb3, vb3, vb2, kb1, vb1, sl_b0, sl_b1, sl_a0, sl_a1, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE(LAG, it, kb0, vb0, vb3, kb2, vb2, sl_a0, sl_a1, sl_b0, sl_b1, 1, 0) ++it; \
        }
        if (lag) {
            RAX_PLOOPS(1)
            RAX_LAG_TAIL()
        } else {
            RAX_PLOOPS(0)
        }
        RAX_WAIT_VMCNT(0);  // the copies past the end land before the workgroup's LDS is reused
#undef RAX_PLOOPS
    } else {
        // prologue: slots of tiles 0 and 1, their copies, the slot of tile 2; tile 0 widened
        // (the younger operations are tile 1's copies and tile 2's slot load); the slot of tile
        // 3 loaded and the copy of tile 2 issued into its emptied staging buffer
        int s8a = 0, s8b = 0;  // slot register sets 0 and 1
        // prologue: slots of tiles 0 and 1, the copy of tile 0, the slot of tile 2, the copy of
        // tile 1, the slot of tile 3 (so that, as in the loop, a tile's copies are followed by
        // one slot load and the next tile's copies); tile 0 widened once its copies have landed
        RAX_VSLOT8(0, s8a)
        if (ntiles > 1) RAX_VSLOT8(1, s8b)
        RAX_COPY8(sk0, sv0, s8a)
        if (ntiles > 2) RAX_VSLOT8(2, s8a)
        if (ntiles > 1) RAX_COPY8(sk1, sv1, s8b)
        if (ntiles > 3) RAX_VSLOT8(3, s8b)
        if (ntiles > 3) {
            RAX_WAIT_VMCNT(4);
        } else if (ntiles > 2) {
            RAX_WAIT_VMCNT(3);
        } else if (ntiles > 1) {
            RAX_WAIT_VMCNT(2);
        } else {
            RAX_WAIT_VMCNT(0);
        }
        RAX_CONVERT8(sk0, sv0, kb0, vb0)
        // Tile T: staging T % 2, bf16 buffer T % 4, slot set T % 2; the first iteration is
        // peeled. Iteration IT copies tile IT+2 (staging and set IT % 2) and loads the slot of
        // tile IT+4 into the same set.
#define RAX_PLOOPS8(LAG)                                                                    \
        RAX_PTILE8(LAG, it, kb0, vb0, vb3, sk1, sv1, sk0, sv0, kb1, vb1, s8a, 1, 0) ++it;    \
        while (it + 4 <= n_full) {                                                          \
            RAX_PTILE8(LAG, it, kb1, vb1, vb0, sk0, sv0, sk1, sv1, kb2, vb2, s8b, 0, 1) ++it; \
            RAX_PTILE8(LAG, it, kb2, vb2, vb1, sk1, sv1, sk0, sv0, kb3, vb3, s8a, 0, 1) ++it; \
            RAX_PTILE8(LAG, it, kb3, vb3, vb2, sk0, sv0, sk1, sv1, kb0, vb0, s8b, 0, 1) ++it; \
            RAX_PTILE8(LAG, it, kb0, vb0, vb3, sk1, sv1, sk0, sv0, kb1, vb1, s8a, 0, 1) ++it; \
        }                                                                                   \
        while (it < ntiles) {                                                               \
            RAX_PTILE8(LAG, it, kb1, vb1, vb0, sk0, sv0, sk1, sv1, kb2, vb2, s8b, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE8(LAG, it, kb2, vb2, vb1, sk1, sv1, sk0, sv0, kb3, vb3, s8a, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE8(LAG, it, kb3, vb3, vb2, sk0, sv0, sk1, sv1, kb0, vb0, s8b, 1, 0) ++it; \
            if (it >= ntiles) break;                                                        \
            RAX_PTILE8(LAG, it, kb0, vb0, vb3, sk1, sv1, sk0, sv0, kb1, vb1, s8a, 1, 0) ++it; \
        }
        if (lag) {
            RAX_PLOOPS8(1)
            RAX_LAG_TAIL()
        } else {
            RAX_PLOOPS8(0)
        }
        RAX_WAIT_VMCNT(0);  // as for bf16 pools: copies past the end land before LDS is reused
#undef RAX_PLOOPS8
    }
    lsum = sum_pair32(lsum + lsum2);
    if (SPL && row_ok) {
        // partial of split sp: the normalised row (fp32) and m + log2(sum)
        const float inv = out_scale / lsum;
        float* prow_ = o_part + (int64_t)sp * total_tokens * Hq * D + qo_row;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(float4*)(prow_ + 32 * dt + 8 * jj + 4 * h2) =
                    make_float4(acc[dt][4 * jj + 0] * inv, acc[dt][4 * jj + 1] * inv,
                                acc[dt][4 * jj + 2] * inv, acc[dt][4 * jj + 3] * inv);
        if (h2 == 0) lse_part[(int64_t)sp * total_tokens * Hq + qo_row / D] = m + __log2f(lsum);
    } else if (row_ok) {
        const float inv = out_scale / lsum;
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
    // Fused store of the ragged suffix: this workgroup writes kv head g of its own tokens'
    // new rows into their pool slots (each (token, kv head) row has exactly one owner). No
    // workgroup of this launch reads those slots: suffix keys come from the new rows, and
    // prefix slots are disjoint from the store slots.
    if constexpr (RAG) {
        // with key splits the last split stores (it always holds a tile; split 0 may not)
        if (store_loc != nullptr && (!SPL || sp == nsplit - 1)) {
            const int nrows = t_last - t0 + 1;
            constexpr int UPR = D / 8;  // 16-byte units per (token, kv head) row
            for (int u = tid; u < nrows * UPR; u += kExtThreads) {
                const int64_t tok = (int64_t)s0 + t0 + u / UPR;
                const int64_t col = (int64_t)g * D * EB + 16 * (u % UPR);
                const int64_t dst = (int64_t)store_loc[tok] * row_bytes + col;
                const int64_t src = tok * row_bytes + col;
                *(uint4*)((char*)k_pool + dst) = *(const uint4*)(k_new + src);
                *(uint4*)((char*)v_pool + dst) = *(const uint4*)(v_new + src);
            }
        }
    }
}
#undef RAX_VSLOTS
#undef RAX_VCOPY
#undef RAX_RADDR
#undef RAX_RISSUE
#undef RAX_QK
#undef RAX_SM
#undef RAX_PEXP
#undef RAX_PV
#undef RAX_VREAD
#undef RAX_PTILE
#undef RAX_COPY8
#undef RAX_VSLOT8
#undef RAX_CONVERT8
#undef RAX_PTILE8
#undef RAX_WIDEN8
#undef RAX_PCOMPUTE
#undef RAX_LAG_TAIL

// Merge of the key splits: one wave per (request, suffix token, q head) row combines the
// nsplit partials, o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) with M the largest lse
// (splits without keys carry lse -inf and weigh 0), and writes the bf16 row.
template <int D>
__global__ __launch_bounds__(256) void extend_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, uint16_t* __restrict__ o,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ extend_start_loc,
    int64_t total_tokens, int32_t max_extend_len, int32_t Hq, int32_t batch, int32_t nsplit) {
    constexpr int PER = D / 64;  // head_dim elements per lane
    const int64_t wq = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = (int)(wq % Hq);
    const int64_t bt = wq / Hq;
    const int b = (int)(bt / max_extend_len);
    const int t = (int)(bt - (int64_t)b * max_extend_len);
    if (b >= batch) return;
    const int s0 = extend_start_loc[b];
    int e = min(extend_lens[b], max_extend_len);
    e = (int)min((int64_t)e, total_tokens - s0);
    if (t >= e) return;
    const int64_t row = (int64_t)(s0 + t) * Hq + h;
    const int64_t plane = total_tokens * Hq;
    // unrolled by 4 so that four splits' loads are in flight together (a row's splits are
    // still added in order)
    float M = -INFINITY;
#pragma unroll 4
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, lse_part[sp * plane + row]);
    float acc[PER] = {};
    float wsum = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < nsplit; ++sp) {
        const float w = fast_exp2(lse_part[sp * plane + row] - M);
        wsum += w;
        const float* pr = o_part + (sp * plane + row) * D + PER * lane;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] += w * pr[k];
    }
    const float inv = 1.f / wsum;
    uint16_t* dst = o + row * D + PER * lane;
    if constexpr (PER == 2) {
        *(uint32_t*)dst = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
        *dst = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xFFFFu);
    }
}

template <int DH, int G, bool OFF32, bool KV8, bool RAG, bool PG, bool SPL>
int launch_g(const AttnArgs& a, hipStream_t stream, int nsplit) {
    const int BQ = kExtBM / (G > 0 ? G : a.n_q_heads / a.n_kv_heads);
    const int tiles = (a.max_extend_len + BQ - 1) / BQ;
    const int pairs = a.batch * a.n_kv_heads;
    // The last pairs % 8 pairs take 2^spread XCDs each (see the kernel).
    const int rem = pairs % kXcds;
    int spread = 0;
    while (rem && (rem << (spread + 1)) <= kXcds) ++spread;
    const int64_t per_xcd = (int64_t)(pairs / kXcds) * tiles + (rem ? ((tiles - 1) >> spread) + 1 : 0);
    const int64_t blocks = per_xcd * kXcds;
    if (blocks <= 0) return 0;
    if (blocks * nsplit > 0x7fffffff) return -1;
    // FP8 pools: the K scale multiplies every score, the V scale every output element.
    const float scale_log2 = a.sm_scale * kLog2e * (KV8 ? a.k_scale : 1.f);
    const float out_scale = KV8 ? a.v_scale : 1.f;
    float* o_part = nullptr;
    float* lse_part = nullptr;
    if constexpr (SPL) {
        o_part = (float*)a.workspace;
        lse_part = (float*)((char*)a.workspace +
                            extend_split_o_bytes(nsplit, a.total_tokens, a.n_q_heads, a.head_dim));
    }
    hipLaunchKernelGGL((extend_kernel<DH, G, OFF32, KV8, RAG, PG, SPL>), dim3((unsigned)(blocks * nsplit)), dim3(kExtThreads),
                       0, stream, (const uint16_t*)a.q, (uint16_t*)a.o, (const char*)a.k_pool,
                       (const char*)a.v_pool, (const char*)a.k_new, (const char*)a.v_new, a.store_loc,
                       a.r2t, a.r2t_stride, a.req_pool_indices,
                       a.prefix_lens, a.extend_lens, a.extend_start_loc, a.total_tokens,
                       a.max_extend_len, a.max_seq_len, a.n_q_heads, a.n_kv_heads, a.batch, tiles,
                       scale_log2, out_scale, a.page_shift, spread, nsplit, o_part, lse_part);
    if constexpr (SPL) {
        if (hipGetLastError() != hipSuccess) return -1;
        const int64_t rows = (int64_t)a.batch * a.max_extend_len * a.n_q_heads;
        hipLaunchKernelGGL((extend_merge_kernel<DH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                           (const float*)o_part, (const float*)lse_part, (uint16_t*)a.o, a.extend_lens,
                           a.extend_start_loc, a.total_tokens, a.max_extend_len, a.n_q_heads, a.batch, nsplit);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int DH, int G, bool OFF32, bool KV8, bool RAG, bool PG>
int launch_g(const AttnArgs& a, hipStream_t stream) {
    return launch_g<DH, G, OFF32, KV8, RAG, PG, false>(a, stream, 1);
}

// Key splits (see extend_splits) where the call's workspace holds their partials; 32-bit
// offsets only.
inline int32_t split_count(const AttnArgs& a) {
    const int32_t S = extend_splits(a.batch, a.n_q_heads, a.n_kv_heads, a.max_extend_len, a.max_seq_len);
    if (S <= 1 || a.workspace == nullptr ||
        a.workspace_bytes < extend_split_workspace(S, a.total_tokens, a.n_q_heads, a.head_dim))
        return 1;
    return S;
}

template <int DH, int G>
int launch_g(const AttnArgs& a, hipStream_t stream) {
    const int32_t S = split_count(a);
    if (a.kv8) {
        if (a.ragged) return -1;
        const bool off8 = pool_fits_32bit_offsets(a.num_slots, a.n_kv_heads, a.head_dim, 1);
        if (off8 && S > 1) {
            if (a.page_shift) return launch_g<DH, G, true, true, false, true, true>(a, stream, S);
            return launch_g<DH, G, true, true, false, false, true>(a, stream, S);
        }
        if (a.page_shift)
            return off8 ? launch_g<DH, G, true, true, false, true>(a, stream)
                        : launch_g<DH, G, false, true, false, true>(a, stream);
        return off8 ? launch_g<DH, G, true, true, false, false>(a, stream)
                    : launch_g<DH, G, false, true, false, false>(a, stream);
    }
    // ragged: the new rows are addressed like pool rows (row index total_tokens - 1 at most)
    const bool off32 = pool_fits_32bit_offsets(a.num_slots, a.n_kv_heads, a.head_dim, 2) &&
                       (!a.ragged || pool_fits_32bit_offsets(a.total_tokens, a.n_kv_heads, a.head_dim, 2));
    if (a.ragged) {
        if (off32 && S > 1) {
            if (a.page_shift) return launch_g<DH, G, true, false, true, true, true>(a, stream, S);
            return launch_g<DH, G, true, false, true, false, true>(a, stream, S);
        }
        if (a.page_shift)
            return off32 ? launch_g<DH, G, true, false, true, true>(a, stream)
                         : launch_g<DH, G, false, false, true, true>(a, stream);
        return off32 ? launch_g<DH, G, true, false, true, false>(a, stream)
                     : launch_g<DH, G, false, false, true, false>(a, stream);
    }
    if (off32 && S > 1) {
        if (a.page_shift) return launch_g<DH, G, true, false, false, true, true>(a, stream, S);
        return launch_g<DH, G, true, false, false, false, true>(a, stream, S);
    }
    if (a.page_shift)
        return off32 ? launch_g<DH, G, true, false, false, true>(a, stream)
                     : launch_g<DH, G, false, false, false, true>(a, stream);
    return off32 ? launch_g<DH, G, true, false, false, false>(a, stream)
                 : launch_g<DH, G, false, false, false, false>(a, stream);
}

// Both head_dims of group size G (each group size is instantiated in its own translation unit,
// extend_g<G>.hip, so that the build compiles them in parallel; G = 0 is the run-time group
// size that serves every other group up to 256).
template <int G>
int launch_extend_group(const AttnArgs& a, hipStream_t stream) {
    if (a.head_dim == 128) return launch_g<128, G>(a, stream);
    if (a.head_dim == 64) return launch_g<64, G>(a, stream);
    return -1;
}

}  // namespace
}  // namespace rax
