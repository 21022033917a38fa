// DECODE attention, bf16: one query per request over its whole cached context.
//
// Each request has one new query; its score row runs over every earlier token, whose K and V
// are gathered from scattered pool slots ("Inside SGLang", Step 3, "Prefill and decode have
// different shapes" and "Paged KV and the kernels that read it"). The step reads every K/V
// byte of the context once and does ~G flops per byte, so it is bound by HBM bandwidth.
//
// Design (gfx950, wave64):
//  * Balanced key stream. A plan lays the requests' contexts end to end, each
//    rounded up to whole 64-key blocks, and cuts that stream into equal ranges of 256..4096
//    keys, one per workgroup, so that one resident round of workgroups (3 per CU over bf16
//    pools, 2 over FP8 pools) covers it:
//    every wave moves the same number of bytes whatever the mix of context lengths. A range
//    may hold the tail of one request and the head of the next; each (request, range) overlap
//    yields one partial (o, lse) in the workspace, and decode_merge_kernel combines a request's
//    partials with log-sum-exp weights. A workgroup's waves are consecutive kv heads (or
//    consecutive sixteen-head parts of them, for groups above 16). For batches up to 1,024
//    requests every split workgroup computes the plan itself (a scan in LDS); larger batches
//    get it from decode_plan_kernel.
//  * The G query heads that share kv head g are the N dimension of 16x16x32 bf16 MFMAs
//    (grouped-query attention: one gathered K/V row feeds all G heads). Heads beyond G are
//    zero padding; MFMA throughput is far above what the bandwidth bound needs. Groups above
//    16 take ceil(G / 16) waves per kv head, 16 query heads each, reading the same rows.
//  * K rows are loaded straight into the MFMA A-operand layout: lane (n = lane%16,
//    kgrp = lane/16) holds 8 consecutive head_dim elements of key n, i.e. 16-byte loads of
//    64 contiguous bytes per key per instruction.
//  * V is needed with keys along the contraction. Each lane loads the 16-byte pieces of 8
//    keys it needs (head_dim range D/16*n .. +D/16) and transposes the 8x8 block in registers
//    (byte permutes), giving the A operand of O^T = V^T P^T. The output row mapping is
//    permuted to d = (D/16)*m + tile so that those loads are contiguous.
//  * Scores S^T come out of the MFMA with the query head as the lane's column, so the
//    softmax running max/sum is per lane; only the max over the four lane groups needs two
//    cross-lane exchanges per iteration (permlane swaps, no LDS). exp2 with sm_scale*log2(e)
//    folded into one multiply.
//  * Iterations of 32 keys over bf16 pools (168 VGPRs) and 64 keys over FP8 pools (164 VGPRs,
//    as many bytes in flight per wave as 32 bf16 keys): 3 waves per SIMD either way.
//  * Key slots: the workgroup's waves read the same keys, so the range's slot numbers are
//    staged in LDS once with global-to-LDS copies; each lane then reads the slots it needs with
//    ds_read, off the memory-counter path of the K/V row loads. Padding keys past a request's
//    end reuse its last valid slot and get -inf scores, so no load leaves the request's slots.
#include <mutex>
#include <type_traits>

#include "librax.h"
#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

namespace {

// Launch-shape constants (overridable at build time for tuning sweeps).
#ifndef RAX_DEC_WAVES
#define RAX_DEC_WAVES 4
#endif
// Split workgroups resident per CU (the register budget: 3 allows 168 VGPRs, 2 allows 256)
// and keys per iteration, for bf16 and for FP8 pools. bf16: 32-key iterations at 3 workgroups
// per CU; FP8: 64-key iterations at 3 per CU (128-key iterations need 2 per CU: 4-7% slower on
// short and mid contexts, 2% faster on the longest).
#ifndef RAX_DEC_WGS_PER_CU
#define RAX_DEC_WGS_PER_CU 3
#endif
#ifndef RAX_DEC_WGS_PER_CU8
#define RAX_DEC_WGS_PER_CU8 3
#endif
#ifndef RAX_DEC_KPI16
#define RAX_DEC_KPI16 32
#endif
#ifndef RAX_DEC_MIN_KEYS
#define RAX_DEC_MIN_KEYS 256
#endif
#ifndef RAX_DEC_NT
#define RAX_DEC_NT 1
#endif
#ifndef RAX_DEC_KPI8
#define RAX_DEC_KPI8 64
#endif
constexpr int kDecWaves = RAX_DEC_WAVES;  // waves (kv heads) per workgroup
constexpr int kDecKeysPerIter = 64;
constexpr int kDecMaxKeys = 4096;  // keys per workgroup range at most (its slots sit in LDS)
constexpr int kDecMaxSegs = kDecMaxKeys / kDecKeysPerIter;  // requests overlapping one range
static_assert(RAX_DEC_MIN_KEYS % kDecKeysPerIter == 0 && RAX_DEC_MIN_KEYS >= kDecKeysPerIter &&
                  RAX_DEC_MIN_KEYS <= kDecMaxKeys,
              "decode ranges must be whole 64-key iterations, at most 4096 keys");
constexpr int kPlanThreads = 1024;
constexpr int kDecFusedBatch = 1024;  // batches up to this size need no separate plan kernel

template <int D>
using VRow = typename std::conditional<D == 128, uint4, uint2>::type;

template <int D, int E>
__device__ __forceinline__ uint4 vcol(const VRow<D> (&r)[8]) {
    return column8<E>(r);
}

// FP8 E4M3 pools ("Inside SGLang", Step 6): 8 (or 4) bytes per K step or V row piece, widened
// to bf16 in registers right before the MFMA (widen8 of 8 bytes is in rax_device.h). The pool
// scales are applied to the scores (K) and to the output (V) instead of to every element.
using ::rax::widen8;
__device__ __forceinline__ uint4 widen8(uint4 x) { return x; }  // bf16 pools: as stored
__device__ __forceinline__ uint2 widen4(uint32_t x) {
    return make_uint2(bf16x2_of_e4m3<false>(x), bf16x2_of_e4m3<true>(x));
}
__device__ __forceinline__ uint2 widen4(uint2 x) { return x; }

// Element types of one K MFMA step (8 head_dim elements) and of a lane's V row piece (DT
// elements), for bf16 or FP8 pools.
// The score contraction runs over head_dim in any order, provided K and Q use the same one.
// With FP8 pools a lane loads 16 contiguous bytes of a K row (two MFMA steps): MFMA step s of
// lane group kg then covers head_dim 16 kg + 64 (s / 2) + 8 (s % 2) .. +8, and the Q operand is
// loaded in that order (bf16 pools: 8 kg + 32 s, one step per 16-byte load).
template <bool KV8>
__device__ __forceinline__ int k_step_elem(int s, int kg) {
    return KV8 ? 16 * kg + 64 * (s >> 1) + 8 * (s & 1) : 8 * kg + 32 * s;
}
__device__ __forceinline__ uint4 k_half(uint4 x, int hi) {  // bf16x8 of 8 E4M3 bytes
    return widen8(hi ? make_uint2(x.z, x.w) : make_uint2(x.x, x.y));
}

template <int D, bool KV8>
struct DecElems {
    using K = uint4;  // one 16-byte load of a K row: 8 bf16 or 16 E4M3 elements
    using V = typename std::conditional<KV8, typename std::conditional<D == 128, uint2, uint32_t>::type,
                                        VRow<D>>::type;
    static constexpr int bytes = KV8 ? 1 : 2;
};
template <int D>
__device__ __forceinline__ VRow<D> widen_v(typename DecElems<D, true>::V x) {
    if constexpr (D == 128) return widen8(x); else return widen4(x);
}
template <int D>
__device__ __forceinline__ VRow<D> widen_v(VRow<D> x) { return x; }

// One K or V row piece (16 or 8 bytes) at byte offset slot * row_bytes + off from a
// wave-uniform base. With one wave per kv head every K/V byte is read once per step, so the
// loads over bf16 pools are marked non-temporal (NT, measured 2-6% faster on the long-context
// batches). When ceil(G / 16) > 1 waves of a workgroup read the same rows, the loads stay
// cached (NT false): the repeats then hit the CU's cache, +29 to +56% for 24 to 48 query heads
// per kv head, where non-temporal loads fetched every repeat from L2. Over FP8 pools (128-byte
// rows) cached loads measured +20% on 64 requests of 512-4,096 tokens and -1% on the longer
// contexts, so they stay cached there too.
template <bool NT, typename T>
__device__ __forceinline__ T load_piece(const char* p) {
    if constexpr (NT) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        if constexpr (sizeof(T) == 16) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
            return __builtin_bit_cast(T, v);
        } else if constexpr (sizeof(T) == 8) {
            const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
            return __builtin_bit_cast(T, v);
        } else {
            return __builtin_nontemporal_load((const uint32_t*)p);
        }
    } else {
        return *(const T*)p;
    }
}

template <bool OFF32, bool NT, typename T>
__device__ __forceinline__ T row_load(const char* base, int slot, uint32_t row_bytes, uint32_t off) {
    if constexpr (OFF32) {
        return load_piece<NT, T>(base + (__umul24((uint32_t)slot, row_bytes) + off));
    } else {
        return load_piece<NT, T>(base + ((uint64_t)(uint32_t)slot * row_bytes + off));
    }
}

// Keys request b occupies in the stream: its valid keys rounded up to whole iterations.
__device__ __forceinline__ int64_t padded_keys(int L) {
    return L > 0 ? (int64_t)((L + kDecKeysPerIter - 1) / kDecKeysPerIter * kDecKeysPerIter) : 0;
}
__device__ __forceinline__ int64_t padded_len(const int32_t* seq_lens, int b, int32_t max_seq_len) {
    return padded_keys(min(seq_lens[b], max_seq_len));
}

// Range length for a stream of T keys: clamp(64 * ceil(T / (64 * n_target)), min, 4096).
__device__ __forceinline__ int64_t range_keys(int64_t T, int32_t n_target) {
    int64_t chunk = (T + n_target - 1) / n_target;
    chunk = (chunk + kDecKeysPerIter - 1) / kDecKeysPerIter * kDecKeysPerIter;
    return min(max(chunk, (int64_t)RAX_DEC_MIN_KEYS), (int64_t)kDecMaxKeys);
}

// One workgroup. Writes P[b] = stream offset of request b (P[B] = stream length T), the range
// length chunk = clamp(64 * ceil(T / (64 * n_target)), RAX_DEC_MIN_KEYS, 4096), the number of
// non-empty ranges, and for each non-empty range w the request its first key belongs to.
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(
    const int32_t* __restrict__ seq_lens, int32_t B, int32_t max_seq_len, int32_t n_target,
    int64_t* __restrict__ meta, int64_t* __restrict__ P, int32_t* __restrict__ first_req) {
    __shared__ int64_t part[kPlanThreads];
    const int t = threadIdx.x;
    const int per = (B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(B, t * per);
    const int b1 = min(B, b0 + per);
    int64_t own = 0;
    for (int b = b0; b < b1; ++b) own += padded_len(seq_lens, b, max_seq_len);
    part[t] = own;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive scan of the thread sums
        const int64_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    const int64_t T = part[kPlanThreads - 1];
    const int64_t chunk = range_keys(T, n_target);
    int64_t run = part[t] - own;
    for (int b = b0; b < b1; ++b) {
        const int64_t len = padded_len(seq_lens, b, max_seq_len);
        P[b] = run;
        for (int64_t w = (run + chunk - 1) / chunk; w * chunk < run + len; ++w) first_req[w] = b;
        run += len;
    }
    if (t == 0) {
        P[B] = T;
        meta[0] = T;
        meta[1] = chunk;
        meta[2] = (T + chunk - 1) / chunk;
    }
}

// A (request, range) overlap: request b, its r2t row, offset of the overlap in the range, its
// length (whole iterations), position of its first key in the request, and the request's
// valid key count.
struct Seg {
    int32_t b, rpi, lo, n, pos0, len;
};

// FUSED (batch <= kDecFusedBatch): every workgroup computes the request offsets itself (a
// scan of the padded lengths in LDS) instead of reading them from decode_plan_kernel, which is
// then not launched; workgroup 0 writes meta and P for the merge kernel.
// PG: r2t is a page table (page size 2^page_shift): position j lives at slot
// r2t[row, j >> page_shift] << page_shift | (j & (2^page_shift - 1)).
// SHR: ceil(G / 16) > 1 waves read the same K/V rows (cached loads, see load_piece).
template <int D, bool OFF32, bool FUSED, bool KV8, bool PG, bool SHR>
__global__ __launch_bounds__(64 * kDecWaves, KV8 ? RAX_DEC_WGS_PER_CU8 : RAX_DEC_WGS_PER_CU) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
    int32_t B, int32_t Hq, int32_t Hkv, int32_t G, int32_t SG, int32_t groups, int32_t n_target,
    float scale_log2, float out_scale, int64_t* __restrict__ meta, int64_t* __restrict__ P,
    const int32_t* __restrict__ first_req, float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t page_shift) {
    constexpr int S = D / 32;   // 32-wide K-dim steps of the score MFMA
    constexpr int DT = D / 16;  // 16-row output tiles; also head_dim elements per lane per V row
    constexpr bool NT = RAX_DEC_NT && !SHR && !KV8;
    __shared__ int32_t slot_lds[kDecMaxKeys + kDecKeysPerIter];
    __shared__ Seg segs[kDecMaxSegs];
    __shared__ int32_t n_seg_lds;

    // Groups of kv heads vary fastest, so the workgroups reading the same keys run together.
    const int grp = blockIdx.x % groups;
    const int w = blockIdx.x / groups;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    int64_t T, chunk, n_active;
    const int64_t* Pr;  // request offsets: LDS (FUSED) or the plan's array
    int b_first;
    // FUSED: request lengths (clamped) and r2t rows, loaded together by the plan below and
    // read again by the request listing from LDS.
    __shared__ int32_t sLen[FUSED ? kDecFusedBatch : 1];
    __shared__ int32_t sRpi[FUSED ? kDecFusedBatch : 1];
    if constexpr (FUSED) {
        constexpr int NT = 64 * kDecWaves;
        __shared__ int64_t sP[kDecFusedBatch + 1];
        __shared__ int64_t wsum[kDecWaves];
        const int t = threadIdx.x;
        const int per = (B + NT - 1) / NT;
        const int c0 = min(B, t * per);
        const int c1 = min(B, c0 + per);
        int64_t own = 0;
        for (int b = c0; b < c1; ++b) {
            const int L = min(seq_lens[b], max_seq_len);
            sLen[b] = L;
            sRpi[b] = rpi[b];
            own += padded_keys(L);
        }
        // inclusive scan of the thread sums: within each wave by shuffles, then over the waves
        int64_t inc = own;
        for (int off = 1; off < kWave; off <<= 1) {
            const int64_t v = __shfl_up(inc, off, kWave);
            if (lane >= off) inc += v;
        }
        if (lane == kWave - 1) wsum[wv] = inc;
        __syncthreads();
        int64_t before = 0;
        T = 0;
        for (int i = 0; i < kDecWaves; ++i) {
            const int64_t ws = wsum[i];
            before += i < wv ? ws : 0;
            T += ws;
        }
        int64_t run = before + inc - own;
        for (int b = c0; b < c1; ++b) {
            sP[b] = run;
            run += padded_keys(sLen[b]);
        }
        if (t == 0) sP[B] = T;
        chunk = range_keys(T, n_target);
        n_active = (T + chunk - 1) / chunk;
        __syncthreads();
        if (blockIdx.x == 0) {
            for (int b = t; b <= B; b += NT) P[b] = sP[b];
            if (t == 0) {
                meta[0] = T;
                meta[1] = chunk;
                meta[2] = n_active;
            }
        }
        if (w >= n_active) return;  // uniform over the workgroup
        // first request of the range: the last b with sP[b] <= s0 (it holds key s0)
        const int64_t s0_ = (int64_t)w * chunk;
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sP[mid] <= s0_) lo = mid; else hi = mid;
        }
        b_first = lo;
        Pr = sP;
    } else {
        T = meta[0];
        chunk = meta[1];
        n_active = meta[2];
        if (w >= n_active) return;  // uniform over the workgroup
        b_first = first_req[w];
        Pr = P;
    }
    const int64_t s0 = (int64_t)w * chunk;
    const int64_t s1 = min(s0 + chunk, T);

    // Wave 0 lists the requests overlapping [s0, s1): they are consecutive from b_first; lane i
    // looks at request wb + i, 64 requests per step (empty requests overlap nothing).
    if (wv == 0) {
        int n_seg = 0;
        for (int wb = b_first; wb < B; wb += kWave) {
            const int bi = wb + lane;
            int64_t pb = s1, pe = s1;
            int rp = 0, len = 0;
            if (bi < B) {
                pb = Pr[bi];
                pe = Pr[bi + 1];
                if constexpr (FUSED) {
                    rp = sRpi[bi];
                    len = sLen[bi];
                } else {
                    rp = rpi[bi];
                    len = min(seq_lens[bi], max_seq_len);
                }
            }
            const bool ov = bi < B && pe > pb && pe > s0 && pb < s1;
            const uint64_t ball = __ballot(ov);
            if (ov) {
                const int64_t a = max(pb, s0);
                const int64_t e = min(pe, s1);
                const int idx = n_seg + __popcll(ball & ((1ull << lane) - 1ull));
                segs[idx] = Seg{bi, rp, (int)(a - s0), (int)(e - a), (int)(a - pb), len};
            }
            n_seg += __popcll(ball);
            if (__shfl((int)(pe >= s1), kWave - 1, kWave)) break;
        }
        if (lane == 0) n_seg_lds = n_seg;
    }
    __syncthreads();
    const int n_seg = n_seg_lds;

    // Stage the range's slot numbers: iteration block j of the range goes to wave j % waves;
    // lane l copies the slot of key l of the block (global-to-LDS, all copies in flight at once).
    for (int si = 0; si < n_seg; ++si) {
        const Seg sg = segs[si];
        const int32_t* row = r2t + (int64_t)sg.rpi * r2t_stride;
        const int j0 = sg.lo / kDecKeysPerIter;
        // With 128-key iterations (FP8 pools) the last one may run 64 keys past the range:
        // stage one more block of slots there (positions clamped to the request, then masked).
        const int nb = sg.n / kDecKeysPerIter + ((KV8 && RAX_DEC_KPI8 > 64 && si == n_seg - 1) ? 1 : 0);
        for (int j = (wv - j0 % kDecWaves + kDecWaves) % kDecWaves; j < nb; j += kDecWaves) {
            const int pos = min(sg.pos0 + j * kDecKeysPerIter + lane, sg.len - 1);
            if constexpr (PG) {
                // the slot is computed from the position's page entry
                slot_lds[sg.lo + j * kDecKeysPerIter + lane] =
                    (row[pos >> page_shift] << page_shift) | (pos & ((1 << page_shift) - 1));
            } else {
                __builtin_amdgcn_global_load_lds(
                    (__attribute__((address_space(1))) void*)(row + pos),
                    (__attribute__((address_space(3))) void*)(slot_lds + sg.lo + j * kDecKeysPerIter),
                    4, 0, 0);
            }
        }
    }
    __syncthreads();

    // Wave v serves kv head g = v / SG and its query heads 16 sub .. 16 sub + 15 (sub = v % SG):
    // groups above 16 split into SG = ceil(G / 16) waves that read the same K/V rows.
    const int v = __builtin_amdgcn_readfirstlane(grp * kDecWaves + wv);
    if (v >= Hkv * SG) return;
    const int g = __builtin_amdgcn_readfirstlane(v / SG);
    const int sub = v - g * SG;
    const int h0 = g * G + 16 * sub;           // first query head of this wave
    const int gw = min(G - 16 * sub, 16);      // query heads of this wave

    const int n16 = lane & 15;
    const int kg = lane >> 4;
    using EL = DecElems<D, KV8>;
    // Keys per iteration (see RAX_DEC_KPI16 / RAX_DEC_KPI8): TT 16-key score tiles, UU 32-key
    // P V steps.
    constexpr int KPI = KV8 ? RAX_DEC_KPI8 : RAX_DEC_KPI16;
    constexpr int TT = KPI / 16;
    constexpr int UU = KPI / 32;
    constexpr uint32_t es = EL::bytes;  // bytes per stored element
    const uint32_t row_bytes = (uint32_t)Hkv * D * es;
    const char* kbase = (const char*)k_pool + (int64_t)g * D * es;  // wave-uniform
    const char* vbase = (const char*)v_pool + (int64_t)g * D * es;
    const uint32_t k_off = 16u * kg;        // this lane's first 16 bytes of a K row
    constexpr int KL = KV8 ? S / 2 : S;     // 16-byte K loads per key
    const uint32_t v_off = es * DT * n16;   // this lane's DT head_dim elements of a V row
    // Columns n16 >= gw are padding: they load a valid head and zero it with a mask (no branch,
    // so the loads stay in flight together).
    const bool q_ok = n16 < gw;
    const uint32_t q_keep = q_ok ? 0xFFFFFFFFu : 0u;

    // Software pipeline over KPI-key iterations: the next iteration's K rows are requested as
    // soon as the score MFMAs have consumed this iteration's, and its V rows as soon as P V has
    // consumed this iteration's, so one iteration of K and V is always in flight. The steady
    // loop is branch-free (the last iteration is peeled), which keeps the memory-counter waits
    // exact: each wait covers only the rows about to be used.
    uint4 kr[TT][KL];
    typename EL::V vr[UU][8];
#define RAX_DEC_SLOTS_K(IT, SK)                                                              \
    _Pragma("unroll") for (int t = 0; t < TT; ++t) SK[t] =                                   \
        slot_lds[lo + (IT) * KPI + 16 * t + n16];
#define RAX_DEC_LOAD_K(SK)                                                                   \
    _Pragma("unroll") for (int t = 0; t < TT; ++t)                                           \
    _Pragma("unroll") for (int s = 0; s < KL; ++s)                                           \
        kr[t][s] = row_load<OFF32, NT, uint4>(kbase, SK[t], row_bytes, k_off + 64u * s);
    // V keys of lane (n16, kg) in block u: 32u + 16h + 4kg + e for h, e in {0,1} x {0..3}.
#define RAX_DEC_LOAD_V(IT)                                                                   \
    _Pragma("unroll") for (int u = 0; u < UU; ++u)                                           \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                          \
        const int4 sv_ =                                                                     \
            *(const int4*)&slot_lds[lo + (IT) * KPI + 32 * u + 16 * h + 4 * kg];             \
        vr[u][4 * h + 0] = row_load<OFF32, NT, typename EL::V>(vbase, sv_.x, row_bytes, v_off); \
        vr[u][4 * h + 1] = row_load<OFF32, NT, typename EL::V>(vbase, sv_.y, row_bytes, v_off); \
        vr[u][4 * h + 2] = row_load<OFF32, NT, typename EL::V>(vbase, sv_.z, row_bytes, v_off); \
        vr[u][4 * h + 3] = row_load<OFF32, NT, typename EL::V>(vbase, sv_.w, row_bytes, v_off); \
    }
#define RAX_DEC_ITER(IT, MORE)                                                               \
    {                                                                                        \
        int sk_[TT];                                                                         \
        if (MORE) { RAX_DEC_SLOTS_K((IT) + 1, sk_) }                                         \
        /* S^T[key][head]: lane holds keys 16t + 4kg + i of head n16. */                     \
        f32x4 st[TT];                                                                        \
        _Pragma("unroll") for (int t = 0; t < TT; ++t) {                                     \
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};                                               \
            _Pragma("unroll") for (int s = 0; s < S; ++s)                                    \
                st[t] = mfma16x16x32(                                                        \
                    as_bf16x8(KV8 ? k_half(kr[t][s >> 1], s & 1) : kr[t][s]), qop[s], st[t]);  \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        if (MORE) { RAX_DEC_LOAD_K(sk_) }                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        float mx = -INFINITY;                                                                \
        _Pragma("unroll") for (int t = 0; t < TT; ++t)                                       \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
            if (!(MORE) && (IT) * KPI + 16 * t + 4 * kg + i >= n_valid)                      \
                st[t][i] = -INFINITY;                                                        \
            mx = fmaxf(mx, st[t][i]);                                                        \
        }                                                                                    \
        mx = max_pair32(max_pair16(mx));                                                     \
        mx *= scale_log2;                                                                    \
        const float m_new = fmaxf(m, mx);                                                    \
        const float alpha = fast_exp2(m - m_new);                                            \
        m = m_new;                                                                           \
        lsum *= alpha;                                                                       \
        _Pragma("unroll") for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;                  \
        float p[TT][4];                                                                      \
        _Pragma("unroll") for (int t = 0; t < TT; ++t)                                       \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
            p[t][i] = fast_exp2(fmaf(st[t][i], scale_log2, -m));                             \
            lsum += p[t][i];                                                                 \
        }                                                                                    \
        /* O^T[d][head] += V^T[d][key] P^T[key][head] per 32-key block. */                   \
        _Pragma("unroll") for (int u = 0; u < UU; ++u) {                                     \
            uint4 pb;                                                                        \
            pb.x = pack_bf16x2(p[2 * u][0], p[2 * u][1]);                                    \
            pb.y = pack_bf16x2(p[2 * u][2], p[2 * u][3]);                                    \
            pb.z = pack_bf16x2(p[2 * u + 1][0], p[2 * u + 1][1]);                            \
            pb.w = pack_bf16x2(p[2 * u + 1][2], p[2 * u + 1][3]);                            \
            const bf16x8 pop = as_bf16x8(pb);                                                \
            VRow<D> vw_[8];                                                                  \
            _Pragma("unroll") for (int j = 0; j < 8; ++j) vw_[j] = widen_v<D>(vr[u][j]);     \
            acc[0] = mfma16x16x32(as_bf16x8(vcol<D, 0>(vw_)), pop, acc[0]);                  \
            acc[1] = mfma16x16x32(as_bf16x8(vcol<D, 1>(vw_)), pop, acc[1]);                \
            acc[2] = mfma16x16x32(as_bf16x8(vcol<D, 2>(vw_)), pop, acc[2]);                \
            acc[3] = mfma16x16x32(as_bf16x8(vcol<D, 3>(vw_)), pop, acc[3]);                \
            if constexpr (DT == 8) {                                                         \
                acc[4] = mfma16x16x32(as_bf16x8(vcol<D, 4>(vw_)), pop, acc[4]);            \
                acc[5] = mfma16x16x32(as_bf16x8(vcol<D, 5>(vw_)), pop, acc[5]);            \
                acc[6] = mfma16x16x32(as_bf16x8(vcol<D, 6>(vw_)), pop, acc[6]);            \
                acc[7] = mfma16x16x32(as_bf16x8(vcol<D, 7>(vw_)), pop, acc[7]);            \
            }                                                                                \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        if (MORE) { RAX_DEC_LOAD_V((IT) + 1) }                                               \
    }

    for (int si = 0; si < n_seg; ++si) {
        const int b = __builtin_amdgcn_readfirstlane(segs[si].b);
        const int lo = __builtin_amdgcn_readfirstlane(segs[si].lo);
        const int n_seg_keys = __builtin_amdgcn_readfirstlane(segs[si].n);
        // Keys of this overlap that count: those of the request (at least one: every 64-key
        // block of a request's padded range starts before its end) and inside the overlap.
        const int n_valid = min(__builtin_amdgcn_readfirstlane(segs[si].len) -
                                    __builtin_amdgcn_readfirstlane(segs[si].pos0),
                                n_seg_keys);
        // Iterations up to the last valid key: only the last one can hold padding keys (which
        // the mask removes), whatever the iteration width.
        const int n_it = (n_valid + KPI - 1) / KPI;

        // B operand of S^T = K Q^T: lane holds Q[head n16][k_step_elem(s, kg) .. +8].
        bf16x8 qop[S];
        {
            const uint16_t* qr = q + ((int64_t)b * Hq + h0 + (q_ok ? n16 : 0)) * D;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                uint4 v = *(const uint4*)(qr + k_step_elem<KV8>(s, kg));
                v.x &= q_keep; v.y &= q_keep; v.z &= q_keep; v.w &= q_keep;
                qop[s] = as_bf16x8(v);
            }
        }
        {
            int sk0[TT];
            RAX_DEC_SLOTS_K(0, sk0)
            RAX_DEC_LOAD_K(sk0)
        }
        RAX_DEC_LOAD_V(0)

        float m = -INFINITY;
        float lsum = 0.f;
        f32x4 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

        int it = 0;
        for (; it + 1 < n_it; ++it) RAX_DEC_ITER(it, true)
        RAX_DEC_ITER(it, false)

        lsum = sum_pair32(sum_pair16(lsum));
        if (q_ok) {
            // Partial of (request b, range w) sits at index b + w: the overlapping pairs form a
            // monotone staircase in (b, w), so b + w never repeats.
            const int64_t pidx = ((int64_t)b + w) * Hq + h0 + n16;
            const float inv = out_scale / lsum;
            float* op = o_part + pidx * D;
            // acc[dt][i] is O^T row 4kg + i, i.e. head_dim DT*(4kg + i) + dt.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4* dst = (float4*)(op + DT * (4 * kg + i));
                dst[0] = make_float4(acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv,
                                     acc[3][i] * inv);
                if constexpr (DT == 8)
                    dst[1] = make_float4(acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv,
                                         acc[7][i] * inv);
            }
            if (kg == 0) lse_part[pidx] = m + __log2f(lsum);
        }
    }
#undef RAX_DEC_ITER
#undef RAX_DEC_SLOTS_K
#undef RAX_DEC_LOAD_K
#undef RAX_DEC_LOAD_V
}

// One wave per (request, q head): o = sum_c 2^(lse_c - M) o_c / sum_c 2^(lse_c - M) over the
// request's partials, one per range its padded key span overlaps. Lane c % 64 holds partial c's
// lse and weight; the o rows of kMergeRows partials are loaded together (the first block goes
// out with the lse loads), so a request's partials cost one memory round trip per block rather
// than one per partial. The rows are accumulated in partial order.
constexpr int kMergeRows = 8;

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, uint16_t* __restrict__ o,
    const int32_t* __restrict__ seq_lens, int32_t max_seq_len, const int64_t* __restrict__ meta,
    const int64_t* __restrict__ P, int32_t Hq, int32_t B) {
    constexpr int PER = D / 64;
    constexpr int U = kMergeRows;
    using Piece = typename std::conditional<PER == 2, float2, float>::type;
    const int wq = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wq >= B * Hq) return;
    const int lane = threadIdx.x & 63;
    const int b = wq / Hq;
    const int h = wq - b * Hq;
    // the length and the plan entries are independent loads: issue them together
    const int L = min(seq_lens[b], max_seq_len);
    const int64_t chunk = meta[1];
    const int64_t pb = P[b], pe = P[b + 1];
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    if (L > 0) {
        const int64_t w0 = pb / chunk;
        const int n = (int)((pe - 1) / chunk - w0) + 1;
        const int64_t first = ((int64_t)b + w0) * Hq + h;  // partial c sits at first + c * Hq
        // Partial c's piece of this lane: o_part[(first + c * Hq) * D + PER * lane ..].
        const Piece* orow = (const Piece*)(o_part + first * D) + lane;
        const int64_t ostep = (int64_t)Hq * D / PER;
        Piece v[U];
        // Rows c .. c + U - 1, indices past the last partial clamped to it (their weight is 0).
        auto load_rows = [&](int c) {
#pragma unroll
            for (int k = 0; k < U; ++k) v[k] = orow[(int64_t)min(c + k, n - 1) * ostep];
        };
        load_rows(0);
        const float lse_own = lane < n ? lse_part[first + (int64_t)lane * Hq] : -INFINITY;
        float M = lse_own;
        for (int c = lane + kWave; c < n; c += kWave) M = fmaxf(M, lse_part[first + (int64_t)c * Hq]);
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) M = wave_max_xor(M, s);
        float wpart = 0.f;
        for (int c0 = 0; c0 < n; c0 += kWave) {
            const int c = c0 + lane;
            const float lc =
                c0 == 0 ? lse_own : (c < n ? lse_part[first + (int64_t)c * Hq] : -INFINITY);
            const float wt = fast_exp2(lc - M);  // 0 in lanes past the last partial
            wpart += wt;
            const int m = min(kWave, n - c0);
            for (int j = 0; j < m; j += U) {
                if (c0 + j > 0) load_rows(c0 + j);
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const float wk =
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j + k));
                    if constexpr (PER == 2) {
                        acc[0] += wk * v[k].x;
                        acc[1] += wk * v[k].y;
                    } else {
                        acc[0] += wk * v[k];
                    }
                }
            }
        }
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) wpart += __shfl_xor(wpart, s, kWave);
        const float inv = 1.f / wpart;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] *= inv;
    }
    uint16_t* dst = o + (int64_t)wq * D + PER * lane;
    if constexpr (PER == 2) {
        *(uint32_t*)dst = pack_bf16x2(acc[0], acc[1]);
    } else {
        *dst = (uint16_t)(pack_bf16x2(acc[0], 0.f) & 0xFFFFu);
    }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int32_t decode_groups(int32_t n_kv_heads) { return (n_kv_heads + kDecWaves - 1) / kDecWaves; }

// Ranges per kv-head group that one resident round of workgroups (256 CUs) covers.
int32_t decode_target(int32_t n_kv_heads, bool kv8) {
    const int32_t resident = 256 * (kv8 ? RAX_DEC_WGS_PER_CU8 : RAX_DEC_WGS_PER_CU);
    const int32_t t = resident / decode_groups(n_kv_heads);
    return t < 1 ? 1 : t;
}

// Workspace sections: meta (3 int64), P (batch + 1 int64), first_req (grid int32), partial o
// (fp32, head_dim each) and lse (fp32) for (batch + grid) * n_q_heads partials.
struct DecLayout {
    size_t meta, P, first, o, lse, total;
};

DecLayout decode_layout(int32_t batch, int32_t grid, int32_t n_q_heads, int32_t head_dim) {
    DecLayout l{};
    const size_t parts = ((size_t)batch + grid) * n_q_heads;
    l.meta = 0;
    l.P = l.meta + 256;
    l.first = l.P + align256(((size_t)batch + 1) * sizeof(int64_t));
    l.o = l.first + align256((size_t)grid * sizeof(int32_t));
    l.lse = l.o + align256(parts * head_dim * sizeof(float));
    l.total = l.lse + parts * sizeof(float);
    return l;
}

// Scratch of the no-allocation DECODE call: the plan and the partials, laid out as the
// workspace. One copy per device, held until the process ends; host code never uses this name
// as an address (it is a host-side stand-in): only the per-device address looked up below.
static __device__ __align__(256) char scratch[RAX_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

void* decode_scratch(hipStream_t stream) {
    int dev = -1;
    if (stream != nullptr) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // each device holds its own copy at its own address: look it up with that device current
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

bool decode_bf16_supported(int32_t group, int32_t head_dim) {
    return group >= 1 && group <= 256 && (head_dim == 64 || head_dim == 128);
}

int32_t decode_wave_heads(int32_t n_q_heads, int32_t n_kv_heads) {
    const int32_t G = n_q_heads / n_kv_heads;
    return n_kv_heads * ((G + 15) / 16);
}

// Ranges per kv-head group the split kernel is launched with: one resident round, or more when
// the longest possible stream (every request at max_seq_len) needs more 4096-key ranges.
// -1 when that would exceed the grid limit.
int32_t decode_grid(int32_t batch, int32_t max_seq_len, int32_t n_kv_heads, bool kv8) {
    const int64_t worst = (int64_t)batch * (((int64_t)max_seq_len + kDecKeysPerIter - 1) /
                                            kDecKeysPerIter * kDecKeysPerIter);
    int64_t n = (worst + kDecMaxKeys - 1) / kDecMaxKeys;
    if (n < decode_target(n_kv_heads, kv8)) n = decode_target(n_kv_heads, kv8);
    if (n * decode_groups(n_kv_heads) > INT32_MAX || n + batch > INT32_MAX) return -1;
    return (int32_t)n;
}

size_t decode_workspace(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, bool kv8) {
    const int32_t grid = decode_grid(batch, max_seq_len, decode_wave_heads(n_q_heads, n_kv_heads), kv8);
    if (grid < 0) return 0;
    return decode_layout(batch, grid, n_q_heads, head_dim).total;
}

int launch_decode_bf16(const AttnArgs& a, hipStream_t stream) {
    const int32_t G = a.n_q_heads / a.n_kv_heads;
    const int32_t SG = (G + 15) / 16;  // waves per kv head (16 query heads each)
    const int32_t wheads = a.n_kv_heads * SG;
    const int32_t groups = decode_groups(wheads);
    const int32_t grid = decode_grid(a.batch, a.max_seq_len, wheads, a.kv8);
    if (grid < 0) return -1;
    const DecLayout l = decode_layout(a.batch, grid, a.n_q_heads, a.head_dim);
    char* ws = (char*)a.workspace;
    int64_t* meta = (int64_t*)(ws + l.meta);
    int64_t* P = (int64_t*)(ws + l.P);
    int32_t* first = (int32_t*)(ws + l.first);
    float* o_part = (float*)(ws + l.o);
    float* lse = (float*)(ws + l.lse);
    const float scale_log2 = a.sm_scale * kLog2e * (a.kv8 ? a.k_scale : 1.f);
    const float out_scale = a.kv8 ? a.v_scale : 1.f;
    const int32_t n_target = decode_target(wheads, a.kv8);
    const bool fused = a.batch <= kDecFusedBatch;
    if (!fused) {
        hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.seq_lens,
                           a.batch, a.max_seq_len, n_target, meta, P, first);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    const dim3 sgrid((uint32_t)grid * (uint32_t)groups);
    const dim3 mgrid((a.batch * a.n_q_heads + 3) / 4);
    const bool off32 = pool_fits_32bit_offsets(a.num_slots, a.n_kv_heads, a.head_dim, a.kv8 ? 1 : 2);
#define RAX_DEC_SPLIT5(DD, OFF, FU, K8, PGT, SH)                                                \
    hipLaunchKernelGGL((decode_split_kernel<DD, OFF, FU, K8, PGT, SH>), sgrid, dim3(64 * kDecWaves), \
                       0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k_pool,                \
                       (const uint16_t*)a.v_pool, a.r2t, a.r2t_stride, a.req_pool_indices,        \
                       a.seq_lens, a.max_seq_len, a.batch, a.n_q_heads, a.n_kv_heads, G, SG,      \
                       groups,                                                                    \
                       n_target, scale_log2, out_scale, meta, P, first, o_part, lse, a.page_shift)
#define RAX_DEC_SPLIT4(DD, OFF, FU, K8, PGT)                                                    \
    do {                                                                                        \
        if (SG > 1) RAX_DEC_SPLIT5(DD, OFF, FU, K8, PGT, true);                                 \
        else RAX_DEC_SPLIT5(DD, OFF, FU, K8, PGT, false);                                       \
    } while (0)
#define RAX_DEC_SPLIT3(DD, OFF, FU)                                                             \
    do {                                                                                        \
        if (a.kv8 && a.page_shift) RAX_DEC_SPLIT4(DD, OFF, FU, true, true);                     \
        else if (a.kv8) RAX_DEC_SPLIT4(DD, OFF, FU, true, false);                               \
        else if (a.page_shift) RAX_DEC_SPLIT4(DD, OFF, FU, false, true);                        \
        else RAX_DEC_SPLIT4(DD, OFF, FU, false, false);                                         \
    } while (0)
#define RAX_DEC_SPLIT(DD, OFF)                                                                  \
    do {                                                                                        \
        if (fused) RAX_DEC_SPLIT3(DD, OFF, true); else RAX_DEC_SPLIT3(DD, OFF, false);          \
    } while (0)
    if (a.head_dim == 128) {
        if (off32) RAX_DEC_SPLIT(128, true); else RAX_DEC_SPLIT(128, false);
        if (hipGetLastError() != hipSuccess) return -1;
        hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, o_part, lse,
                           (uint16_t*)a.o, a.seq_lens, a.max_seq_len, meta, P, a.n_q_heads, a.batch);
    } else {
        if (off32) RAX_DEC_SPLIT(64, true); else RAX_DEC_SPLIT(64, false);
        if (hipGetLastError() != hipSuccess) return -1;
        hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, o_part, lse,
                           (uint16_t*)a.o, a.seq_lens, a.max_seq_len, meta, P, a.n_q_heads, a.batch);
    }
#undef RAX_DEC_SPLIT
#undef RAX_DEC_SPLIT3
#undef RAX_DEC_SPLIT4
#undef RAX_DEC_SPLIT5
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace rax
