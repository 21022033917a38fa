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
//    row, 16-byte loads, 16 lanes per row: coalesced) into registers one tile ahead, then store
//    them to LDS: K row-major [key][d], V transposed [d][key] (4 keys x 8 head_dim elements
//    per thread, transposed with register byte permutes). Both LDS arrays are XOR-swizzled in
//    16-byte units so that the MFMA operand reads (8 consecutive rows per 8 lanes) and the
//    stores are free or nearly free of bank conflicts.
//  * S^T = K Q^T with 32x32x16 bf16 MFMAs: keys are the M dimension (read from LDS), query
//    rows the N dimension (Q stays in registers for the whole key loop). The C layout puts
//    one query row per lane column, so the row max/sum are per lane plus one exchange with
//    the other half-wave.
//  * O^T = V^T P^T, also 32x32x16: P^T is the score C fragment converted to bf16 in place
//    (the key order inside each 16-key step is a fixed bit permutation that the V^T layout in
//    LDS follows), so P never leaves registers.
//  * Causal mask only on the tiles that cross the diagonal; keys past the last visible key of
//    the workgroup reuse a valid slot and are masked, so no load leaves the request's slots.
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

__device__ __forceinline__ int swz_k(int key, int unit) { return unit ^ (key & 7); }
__device__ __forceinline__ int swz_v(int d, int unit) { return unit ^ ((d ^ (d >> 3)) & 7); }

// Key offset (within a 16-key MFMA step) held at k-slot q of the P^T fragment: bits 2 and 3
// swapped. The map is its own inverse.
__device__ __forceinline__ int swap23(int q) { return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1); }

template <int G>
__global__ __launch_bounds__(kExtThreads, 2) void extend_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ r2t, int64_t r2t_stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ extend_start_loc,
    int64_t total_tokens, int32_t max_extend_len, int32_t max_seq_len, int32_t Hq, int32_t Hkv,
    int32_t batch, int32_t tiles, float scale_log2) {
    constexpr int D = kExtD;
    constexpr int BQ = kExtBM / G;  // tokens per workgroup

    __shared__ uint4 k_lds[kExtBN * 16];  // [key][16 units of 8 bf16]
    __shared__ uint4 vt_lds[D * 8];       // [d][8 units of 8 keys]

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
    const int64_t pool_row = (int64_t)Hkv * D;
    const uint16_t* kbase = k_pool + (int64_t)g * D;
    const uint16_t* vbase = v_pool + (int64_t)g * D;

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

    // ---- cooperative gather roles
    const int seg = tid & 15;  // 16-byte unit of head_dim (8 elements)
    const int grp = tid >> 4;  // 0..15
    // K: keys grp + 16 i; V: keys 4 grp + i (i = 0..3)
    uint4 kst[4], vst[4];
    auto gather = [&](int j0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kj = min(j0 + grp + 16 * i, kend - 1);
            const int vj = min(j0 + 4 * grp + i, kend - 1);
            const int ks = row[kj];
            const int vs = row[vj];
            kst[i] = *(const uint4*)(kbase + (int64_t)ks * pool_row + 8 * seg);
            vst[i] = *(const uint4*)(vbase + (int64_t)vs * pool_row + 8 * seg);
        }
    };
    // V^T position of key 4*grp + i: 16-key step (grp / 4), offset swap23(4 (grp % 4) + i).
    const int vpos0 = 16 * (grp >> 2) + swap23(4 * (grp & 3));
    const int vunit = vpos0 >> 3;
    const int vhalf = (vpos0 >> 2) & 1;
    auto to_lds = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = grp + 16 * i;
            k_lds[key * 16 + swz_k(key, seg)] = kst[i];
        }
        uint2* vt2 = (uint2*)vt_lds;
#define RAX_VT_STORE(DD)                                                                        \
        {                                                                                       \
            const int d = 8 * seg + DD;                                                         \
            uint2 w;                                                                            \
            w.x = half_of<DD>(vst[0]) | (half_of<DD>(vst[1]) << 16);                            \
            w.y = half_of<DD>(vst[2]) | (half_of<DD>(vst[3]) << 16);                            \
            vt2[(d * 8 + swz_v(d, vunit)) * 2 + vhalf] = w;                                     \
        }
        RAX_VT_STORE(0) RAX_VT_STORE(1) RAX_VT_STORE(2) RAX_VT_STORE(3)
        RAX_VT_STORE(4) RAX_VT_STORE(5) RAX_VT_STORE(6) RAX_VT_STORE(7)
#undef RAX_VT_STORE
    };

    float m = -INFINITY;
    float lsum = 0.f;
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    const int last_q = p + t;  // last key position this row may see
    const int diag_from = p + t0;  // tiles whose last key exceeds this need the mask
    const int ntiles = (kend + kExtBN - 1) / kExtBN;

    gather(0);
    for (int it = 0; it < ntiles; ++it) {
        const int j0 = it * kExtBN;
        __syncthreads();  // previous tile's LDS reads are done
        to_lds();
        __syncthreads();
        if (it + 1 < ntiles) gather(j0 + kExtBN);

        // S^T: two 32-key M blocks
        f32x16 st[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st[mb][i] = 0.f;
            const int key = 32 * mb + col;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const uint4 a = k_lds[key * 16 + swz_k(key, 2 * s + h2)];
                st[mb] = mfma32x32x16(as_bf16x8(a), qop[s], st[mb]);
            }
        }

        // scale, mask, running max. st[mb][4 jj + i] is key 32 mb + 8 jj + 4 h2 + i.
        const bool need_mask = j0 + kExtBN - 1 > diag_from;
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = st[mb][4 * jj + i] * scale_log2;
                    if (need_mask) {
                        const int key = j0 + 32 * mb + 8 * jj + 4 * h2 + i;
                        x = key <= last_q ? x : -INFINITY;
                    }
                    st[mb][4 * jj + i] = x;
                    mx = fmaxf(mx, x);
                }
        mx = wave_max_xor(mx, 32);
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;

        // P^T fragments: 16-key step kk uses st[kk / 2][8 (kk % 2) .. +8].
        uint4 pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pv[j] = fast_exp2(st[kk >> 1][8 * (kk & 1) + j] - m);
                lsum += pv[j];
            }
            pf[kk].x = pack_bf16x2(pv[0], pv[1]);
            pf[kk].y = pack_bf16x2(pv[2], pv[3]);
            pf[kk].z = pack_bf16x2(pv[4], pv[5]);
            pf[kk].w = pack_bf16x2(pv[6], pv[7]);
        }

        // O^T[d][row] += V^T[d][keys] P^T[keys][row]
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int d = 32 * dt + col;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4 a = vt_lds[d * 8 + swz_v(d, 2 * kk + h2)];
                acc[dt] = mfma32x32x16(as_bf16x8(a), as_bf16x8(pf[kk]), acc[dt]);
            }
        }
    }

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

template <int G>
int launch_g(const AttnArgs& a, hipStream_t stream) {
    constexpr int BQ = kExtBM / G;
    const int tiles = (a.max_extend_len + BQ - 1) / BQ;
    const int pairs = a.batch * a.n_kv_heads;
    const int64_t blocks = (int64_t)((pairs + kXcds - 1) / kXcds) * kXcds * tiles;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL(extend_kernel<G>, dim3((unsigned)blocks), dim3(kExtThreads), 0, stream,
                       (const uint16_t*)a.q, (uint16_t*)a.o, (const uint16_t*)a.k_pool,
                       (const uint16_t*)a.v_pool, a.r2t, a.r2t_stride, a.req_pool_indices,
                       a.prefix_lens, a.extend_lens, a.extend_start_loc, a.total_tokens,
                       a.max_extend_len, a.max_seq_len, a.n_q_heads, a.n_kv_heads, a.batch, tiles,
                       a.sm_scale * kLog2e);
    return hipGetLastError() == hipSuccess ? 0 : -1;
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
