// DECODE attention, bf16: one query per request over its whole cached context.
//
// Each request has one new query; its score row runs over every earlier token, whose K and V
// are gathered from scattered pool slots ("Inside SGLang", Step 3, "Prefill and decode have
// different shapes" and "Paged KV and the kernels that read it"). The step reads every K/V
// byte of the context once and does ~G flops per byte, so it is bound by HBM bandwidth.
//
// Design (gfx950, wave64):
//  * split-K: a wave owns (request b, kv head g, key chunk c). Chunks are sized on the host so
//    that the grid holds thousands of waves; partial (o, lse) go to a workspace and
//    decode_merge_kernel combines them with the usual log-sum-exp weights.
//  * The G query heads that share kv head g are the N dimension of 16x16x32 bf16 MFMAs
//    (grouped-query attention: one gathered K/V row feeds all G heads). Heads beyond G are
//    zero padding; MFMA throughput is far above what the bandwidth bound needs.
//  * No LDS. K rows are loaded straight into the MFMA A-operand layout: lane (n = lane%16,
//    kgrp = lane/16) holds 8 consecutive head_dim elements of key n, i.e. 16-byte loads of
//    64 contiguous bytes per key per instruction.
//  * V is needed with keys along the contraction. Each lane loads the 16-byte pieces of 8
//    keys it needs (head_dim range D/16*n .. +D/16) and transposes the 8x8 block in registers
//    (byte permutes), giving the A operand of O^T = V^T P^T. The output row mapping is
//    permuted to d = (D/16)*m + tile so that those loads are contiguous.
//  * Scores S^T come out of the MFMA with the query head as the lane's column, so the
//    softmax running max/sum is per lane; only the max over the four lane groups needs two
//    cross-lane exchanges per 64 keys. exp2 with sm_scale*log2(e) folded into one multiply.
//  * Key slots: the workgroup's waves (kv heads) read the same keys, so the split's slot numbers
//    are staged in LDS once with coalesced loads; each lane then reads the slots it needs with
//    ds_read, off the memory-counter path of the K/V row loads. Keys past the split end reuse the
//    last valid key's slot and get -inf scores, so no load ever leaves the request's valid slots.
//  * Each request's context is cut into ceil(L / chunk) nearly equal splits, so split lengths
//    differ by less than 2x across requests and no split is a short remainder.
#include <type_traits>

#include "rax_device.h"
#include "rax_launch.h"

namespace rax {

namespace {

// Launch-shape constants (overridable at build time for tuning sweeps).
#ifndef RAX_DEC_WAVES
#define RAX_DEC_WAVES 4
#endif
#ifndef RAX_DEC_TARGET_WAVES
#define RAX_DEC_TARGET_WAVES 2048
#endif
#ifndef RAX_DEC_MIN_CHUNK
#define RAX_DEC_MIN_CHUNK 256
#endif
#ifndef RAX_DEC_FIXED_CHUNK
#define RAX_DEC_FIXED_CHUNK 0
#endif
constexpr int kDecWaves = RAX_DEC_WAVES;  // waves (kv heads) per workgroup
constexpr int kDecKeysPerIter = 64;
constexpr int kDecMaxChunk = 4096;  // keys per split, before the 64-key rounding of split edges
static_assert(RAX_DEC_MIN_CHUNK % kDecKeysPerIter == 0 && RAX_DEC_MIN_CHUNK >= 256 &&
                  RAX_DEC_MIN_CHUNK <= kDecMaxChunk,
              "decode chunks must be multiples of 64 in [256, 4096] so that no split is empty");

template <int D>
using VRow = typename std::conditional<D == 128, uint4, uint2>::type;

template <int D, int E>
__device__ __forceinline__ uint4 vcol(const VRow<D> (&r)[8]) {
    return column8<E>(r);
}

#ifndef RAX_DEC_NT
#define RAX_DEC_NT 0
#endif

// One K or V row piece (16 or 8 bytes) at byte offset slot * row_bytes + off from a
// wave-uniform base. Every K/V byte is read once per step, so the loads can be marked
// non-temporal (RAX_DEC_NT).
template <typename T>
__device__ __forceinline__ T load_piece(const char* p) {
    if constexpr (RAX_DEC_NT) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        if constexpr (sizeof(T) == 16) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
            return __builtin_bit_cast(T, v);
        } else {
            const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
            return __builtin_bit_cast(T, v);
        }
    } else {
        return *(const T*)p;
    }
}

template <bool OFF32, typename T>
__device__ __forceinline__ T row_load(const char* base, int slot, uint32_t row_bytes, uint32_t off) {
    if constexpr (OFF32) {
        return load_piece<T>(base + (__umul24((uint32_t)slot, row_bytes) + off));
    } else {
        return load_piece<T>(base + ((uint64_t)(uint32_t)slot * row_bytes + off));
    }
}

// Edges of split c when a context of L keys is cut into ns nearly equal splits: multiples of the
// 64-key iteration except the final end. With ns = ceil(L / chunk) and chunk >= 256 every split
// holds more than 64 and fewer than chunk + 64 keys.
__device__ __forceinline__ int split_edge(int c, int L, int ns) {
    return c >= ns ? L : kDecKeysPerIter * (int)(((int64_t)c * L) / ((int64_t)kDecKeysPerIter * ns));
}

template <int D, bool OFF32>
__global__ __launch_bounds__(64 * kDecWaves, 8 / kDecWaves) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
    int32_t Hq, int32_t Hkv, int32_t G, int32_t chunk, int32_t num_splits, float scale_log2,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
    constexpr int S = D / 32;   // 32-wide K-dim steps of the score MFMA
    constexpr int DT = D / 16;  // 16-row output tiles; also head_dim elements per lane per V row
    __shared__ int32_t slot_lds[kDecMaxChunk + kDecKeysPerIter];

    const int c = blockIdx.x;
    const int b = blockIdx.z;
    const int L = min(seq_lens[b], max_seq_len);
    const int ns = L > 0 ? (L + chunk - 1) / chunk : 0;
    if (c >= ns) return;  // uniform over the workgroup
    const int k0 = split_edge(c, L, ns);
    const int nk = split_edge(c + 1, L, ns) - k0;
    const int n_it = (nk + kDecKeysPerIter - 1) / kDecKeysPerIter;

    // The workgroup's kv heads read the same keys: stage the split's slot numbers once, padded
    // to whole iterations with the last valid slot so that every row load stays in the request.
    // Global-to-LDS copies (lane l of a wave writes dword l of its 64-slot block), so all of a
    // wave's copies are in flight at once; the barrier waits for them.
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    {
        const int32_t* row = r2t + (int64_t)rpi[b] * r2t_stride + k0;
        for (int j = wv; j < n_it; j += kDecWaves)
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void*)(row + min(j * kDecKeysPerIter + lane, nk - 1)),
                (__attribute__((address_space(3))) void*)(slot_lds + j * kDecKeysPerIter), 4, 0, 0);
    }
    __syncthreads();

    const int g = __builtin_amdgcn_readfirstlane(blockIdx.y * kDecWaves + wv);
    if (g >= Hkv) return;

    const int n16 = lane & 15;
    const int kg = lane >> 4;
    const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
    const char* kbase = (const char*)k_pool + (int64_t)g * D * 2;  // wave-uniform
    const char* vbase = (const char*)v_pool + (int64_t)g * D * 2;
    const uint32_t k_off = 16u * kg;       // this lane's 8 head_dim elements of a K row
    const uint32_t v_off = 2u * DT * n16;  // this lane's DT head_dim elements of a V row

    // B operand of S^T = K Q^T: lane holds Q[head n16][32 s + 8 kg .. +8].
    bf16x8 qop[S];
    {
        // Columns n16 >= G are padding: load a valid head and zero it with a mask (no branch, so
        // the four loads stay in flight together).
        const bool ok = n16 < G;
        const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
        const uint16_t* qr = q + ((int64_t)b * Hq + (int64_t)g * G + (ok ? n16 : 0)) * D + 8 * kg;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            uint4 v = *(const uint4*)(qr + 32 * s);
            v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
            qop[s] = as_bf16x8(v);
        }
    }

    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over 64-key iterations: the next iteration's K rows are requested as
    // soon as the score MFMAs have consumed this iteration's, and its V rows as soon as P V has
    // consumed this iteration's, so one iteration of K and V is always in flight. The steady
    // loop is branch-free (the last iteration is peeled), which keeps the memory-counter waits
    // exact: each wait covers only the rows about to be used.
    uint4 kr[4][S];
    VRow<D> vr[2][8];
#define RAX_DEC_SLOTS_K(IT, SK)                                                              \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) SK[t] = slot_lds[(IT) * kDecKeysPerIter + 16 * t + n16];
#define RAX_DEC_LOAD_K(SK)                                                                   \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                            \
    _Pragma("unroll") for (int s = 0; s < S; ++s)                                            \
        kr[t][s] = row_load<OFF32, uint4>(kbase, SK[t], row_bytes, k_off + 64u * s);
    // V keys of lane (n16, kg) in block u: 32u + 16h + 4kg + e for h, e in {0,1} x {0..3}.
#define RAX_DEC_LOAD_V(IT)                                                                   \
    _Pragma("unroll") for (int u = 0; u < 2; ++u)                                            \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                          \
        const int4 sv_ =                                                                     \
            *(const int4*)&slot_lds[(IT) * kDecKeysPerIter + 32 * u + 16 * h + 4 * kg];      \
        vr[u][4 * h + 0] = row_load<OFF32, VRow<D>>(vbase, sv_.x, row_bytes, v_off);         \
        vr[u][4 * h + 1] = row_load<OFF32, VRow<D>>(vbase, sv_.y, row_bytes, v_off);         \
        vr[u][4 * h + 2] = row_load<OFF32, VRow<D>>(vbase, sv_.z, row_bytes, v_off);         \
        vr[u][4 * h + 3] = row_load<OFF32, VRow<D>>(vbase, sv_.w, row_bytes, v_off);         \
    }
#define RAX_DEC_ITER(IT, MORE)                                                               \
    {                                                                                        \
        /* S^T[key][head]: lane holds keys 16t + 4kg + i of head n16. */                     \
        int sk_[4];                                                                          \
        if (MORE) { RAX_DEC_SLOTS_K((IT) + 1, sk_) }                                         \
        f32x4 st[4];                                                                         \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                      \
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};                                               \
            _Pragma("unroll") for (int s = 0; s < S; ++s)                                    \
                st[t] = mfma16x16x32(as_bf16x8(kr[t][s]), qop[s], st[t]);                    \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        if (MORE) { RAX_DEC_LOAD_K(sk_) }                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        float mx = -INFINITY;                                                                \
        _Pragma("unroll") for (int t = 0; t < 4; ++t)                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
            if (!(MORE) && (IT) * kDecKeysPerIter + 16 * t + 4 * kg + i >= nk)               \
                st[t][i] = -INFINITY;                                                        \
            mx = fmaxf(mx, st[t][i]);                                                        \
        }                                                                                    \
        mx = wave_max_xor(mx, 16);                                                           \
        mx = wave_max_xor(mx, 32);                                                           \
        mx *= scale_log2;                                                                    \
        const float m_new = fmaxf(m, mx);                                                    \
        const float alpha = fast_exp2(m - m_new);                                            \
        m = m_new;                                                                           \
        lsum *= alpha;                                                                       \
        _Pragma("unroll") for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;                  \
        float p[4][4];                                                                       \
        _Pragma("unroll") for (int t = 0; t < 4; ++t)                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
            p[t][i] = fast_exp2(fmaf(st[t][i], scale_log2, -m));                             \
            lsum += p[t][i];                                                                 \
        }                                                                                    \
        /* O^T[d][head] += V^T[d][key] P^T[key][head] per 32-key block. */                   \
        _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                      \
            uint4 pb;                                                                        \
            pb.x = pack_bf16x2(p[2 * u][0], p[2 * u][1]);                                    \
            pb.y = pack_bf16x2(p[2 * u][2], p[2 * u][3]);                                    \
            pb.z = pack_bf16x2(p[2 * u + 1][0], p[2 * u + 1][1]);                            \
            pb.w = pack_bf16x2(p[2 * u + 1][2], p[2 * u + 1][3]);                            \
            const bf16x8 pop = as_bf16x8(pb);                                                \
            acc[0] = mfma16x16x32(as_bf16x8(vcol<D, 0>(vr[u])), pop, acc[0]);                \
            acc[1] = mfma16x16x32(as_bf16x8(vcol<D, 1>(vr[u])), pop, acc[1]);                \
            acc[2] = mfma16x16x32(as_bf16x8(vcol<D, 2>(vr[u])), pop, acc[2]);                \
            acc[3] = mfma16x16x32(as_bf16x8(vcol<D, 3>(vr[u])), pop, acc[3]);                \
            if constexpr (DT == 8) {                                                         \
                acc[4] = mfma16x16x32(as_bf16x8(vcol<D, 4>(vr[u])), pop, acc[4]);            \
                acc[5] = mfma16x16x32(as_bf16x8(vcol<D, 5>(vr[u])), pop, acc[5]);            \
                acc[6] = mfma16x16x32(as_bf16x8(vcol<D, 6>(vr[u])), pop, acc[6]);            \
                acc[7] = mfma16x16x32(as_bf16x8(vcol<D, 7>(vr[u])), pop, acc[7]);            \
            }                                                                                \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        if (MORE) { RAX_DEC_LOAD_V((IT) + 1) }                                               \
    }

    {
        int sk0[4];
        RAX_DEC_SLOTS_K(0, sk0)
        RAX_DEC_LOAD_K(sk0)
    }
    RAX_DEC_LOAD_V(0)
    int it = 0;
    for (; it + 1 < n_it; ++it) RAX_DEC_ITER(it, true)
    RAX_DEC_ITER(it, false)
#undef RAX_DEC_ITER
#undef RAX_DEC_SLOTS_K
#undef RAX_DEC_LOAD_K
#undef RAX_DEC_LOAD_V

    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    if (n16 < G) {
        const int h = g * G + n16;
        const int64_t pidx = ((int64_t)b * Hq + h) * num_splits + c;
        const float inv = 1.f / lsum;
        float* op = o_part + pidx * D;
        // acc[dt][i] is O^T row 4kg + i, i.e. head_dim DT*(4kg + i) + dt.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4* dst = (float4*)(op + DT * (4 * kg + i));
            dst[0] = make_float4(acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv);
            if constexpr (DT == 8)
                dst[1] = make_float4(acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv, acc[7][i] * inv);
        }
        if (kg == 0) lse_part[pidx] = m + __log2f(lsum);
    }
}

// One wave per (request, q head): o = sum_c 2^(lse_c - M) o_c / sum_c 2^(lse_c - M).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           uint16_t* __restrict__ o,
                                                           const int32_t* __restrict__ seq_lens,
                                                           int32_t max_seq_len, int32_t chunk,
                                                           int32_t num_splits, int32_t Hq,
                                                           int32_t B) {
    constexpr int PER = D / 64;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= B * Hq) return;
    const int lane = threadIdx.x & 63;
    const int b = w / Hq;
    const int L = min(seq_lens[b], max_seq_len);
    const int nc = L > 0 ? min((L + chunk - 1) / chunk, num_splits) : 0;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    if (nc > 0) {
        const float* lp = lse_part + (int64_t)w * num_splits;
        float M = -INFINITY;
        for (int c = lane; c < nc; c += kWave) M = fmaxf(M, lp[c]);
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) M = wave_max_xor(M, s);
        float wsum = 0.f;
        const float* op = o_part + (int64_t)w * num_splits * D + PER * lane;
        for (int c = 0; c < nc; ++c) {
            const float wt = fast_exp2(lp[c] - M);
            wsum += wt;
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] += wt * op[(int64_t)c * D + k];
        }
        const float inv = 1.f / wsum;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] *= inv;
    }
    uint16_t* dst = o + (int64_t)w * D + PER * lane;
    if constexpr (PER == 2) {
        *(uint32_t*)dst = pack_bf16x2(acc[0], acc[1]);
    } else {
        *dst = (uint16_t)(pack_bf16x2(acc[0], 0.f) & 0xFFFFu);
    }
}

}  // namespace

bool decode_bf16_supported(int32_t group, int32_t head_dim) {
    return group >= 1 && group <= 16 && (head_dim == 64 || head_dim == 128);
}

// Keys per split: enough splits that batch * n_kv_heads * splits is in the thousands of waves
// (256 CUs), in multiples of the 64-key iteration, between RAX_DEC_MIN_CHUNK and 4096 keys.
int32_t decode_chunk(int32_t batch, int32_t max_seq_len, int32_t n_kv_heads) {
    static_assert(RAX_DEC_FIXED_CHUNK == 0 || (RAX_DEC_FIXED_CHUNK % kDecKeysPerIter == 0 &&
                                               RAX_DEC_FIXED_CHUNK >= 256 &&
                                               RAX_DEC_FIXED_CHUNK <= kDecMaxChunk),
                  "fixed decode chunk must be a multiple of 64 in [256, 4096]");
    if (RAX_DEC_FIXED_CHUNK > 0) return RAX_DEC_FIXED_CHUNK;
    const int64_t units = (int64_t)batch * n_kv_heads;
    const int64_t target = RAX_DEC_TARGET_WAVES;
    int64_t want = units > 0 ? ((int64_t)max_seq_len * units + target - 1) / target : RAX_DEC_MIN_CHUNK;
    want = (want + kDecKeysPerIter - 1) / kDecKeysPerIter * kDecKeysPerIter;
    if (want < RAX_DEC_MIN_CHUNK) want = RAX_DEC_MIN_CHUNK;
    if (want > kDecMaxChunk) want = kDecMaxChunk;
    return (int32_t)want;
}

int32_t decode_splits(int32_t batch, int32_t max_seq_len, int32_t n_kv_heads) {
    const int32_t ck = decode_chunk(batch, max_seq_len, n_kv_heads);
    const int32_t n = (max_seq_len + ck - 1) / ck;
    return n < 1 ? 1 : n;
}

size_t decode_workspace(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim) {
    const size_t ns = (size_t)decode_splits(batch, max_seq_len, n_kv_heads);
    const size_t rows = (size_t)batch * n_q_heads * ns;
    // o partials (fp32, head_dim each), then one lse per partial; 256-byte aligned sections.
    const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) / 256 * 256;
    return o_bytes + rows * sizeof(float);
}

int launch_decode_bf16(const AttnArgs& a, hipStream_t stream) {
    const int32_t G = a.n_q_heads / a.n_kv_heads;
    const int32_t chunk = decode_chunk(a.batch, a.max_seq_len, a.n_kv_heads);
    const int32_t ns = decode_splits(a.batch, a.max_seq_len, a.n_kv_heads);
    const size_t rows = (size_t)a.batch * a.n_q_heads * ns;
    float* o_part = (float*)a.workspace;
    float* lse = (float*)((char*)a.workspace + (rows * a.head_dim * sizeof(float) + 255) / 256 * 256);
    const float scale_log2 = a.sm_scale * kLog2e;
    dim3 grid(ns, (a.n_kv_heads + kDecWaves - 1) / kDecWaves, a.batch);
    dim3 mgrid((a.batch * a.n_q_heads + 3) / 4);
    const bool off32 = pool_fits_32bit_offsets(a.num_slots, a.n_kv_heads, a.head_dim, 2);
#define RAX_DEC_SPLIT(DD, OFF)                                                                  \
    hipLaunchKernelGGL((decode_split_kernel<DD, OFF>), grid, dim3(64 * kDecWaves), 0, stream,     \
                       (const uint16_t*)a.q, (const uint16_t*)a.k_pool, (const uint16_t*)a.v_pool,  \
                       a.r2t, a.r2t_stride, a.req_pool_indices, a.seq_lens, a.max_seq_len,         \
                       a.n_q_heads, a.n_kv_heads, G, chunk, ns, scale_log2, o_part, lse)
    if (a.head_dim == 128) {
        if (off32) RAX_DEC_SPLIT(128, true); else RAX_DEC_SPLIT(128, false);
        if (hipGetLastError() != hipSuccess) return -1;
        hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, o_part, lse,
                           (uint16_t*)a.o, a.seq_lens, a.max_seq_len, chunk, ns, a.n_q_heads, a.batch);
    } else {
        if (off32) RAX_DEC_SPLIT(64, true); else RAX_DEC_SPLIT(64, false);
        if (hipGetLastError() != hipSuccess) return -1;
        hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, o_part, lse,
                           (uint16_t*)a.o, a.seq_lens, a.max_seq_len, chunk, ns, a.n_q_heads, a.batch);
    }
#undef RAX_DEC_SPLIT
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace rax
