// Debug checks of the device-side contracts of the librax calls: the index arrays the attention
// and store kernels trust (slots, page entries, request rows, lengths) are read here, only
// inside the bounds the host arguments give, and every entry that breaks a contract is counted
// per kind in a caller-given int32 array. Nothing is dereferenced through an index before that
// index has been checked, so a bad entry is counted and never followed.
//
//  * Store slots (kv_store's loc, the ragged call's store_loc): out of [0, num_slots), or
//    equal to an earlier entry. Repeats are found with one bit per pool slot in the caller's
//    workspace (atomic OR; the entry that finds its bit already set counts), cleared by a fill
//    kernel first.
//  * Requests (one workgroup each): lengths and start against the host maxima, the request row
//    against the table's row count, then every position the call reads: its slot (token table)
//    or page entry (page table) inside the pool, and for the ragged call with a store, not one
//    of the slots that call stores to.
#include "rax_device.h"
#include "rax_launch.h"
#include "rax_check.h"

namespace rax {

namespace {

constexpr int kChkThreads = 256;

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Adds the number of lanes of this wave for which `bad` holds to counts[item]: one atomic per
// wave, issued by the lowest such lane.
__device__ __forceinline__ void count_wave(int32_t* counts, int item, bool bad) {
    const uint64_t m = __ballot(bad);
    if (bad && (int)(threadIdx.x & 63) == __builtin_ctzll(m))
        atomicAdd(counts + item, (int32_t)__popcll(m));
}

__global__ void mark_slots_kernel(const int32_t* __restrict__ loc, int64_t n, int64_t num_slots,
                                  uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts) {
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x; i0 < n; i0 += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = i0 + threadIdx.x;
        bool bad = false, dup = false;
        if (i < n) {
            const int64_t s = loc[i];
            bad = s < 0 || s >= num_slots;
            if (!bad) {
                const uint32_t bit = 1u << (s & 31);
                dup = (atomicOr(bitmap + (s >> 5), bit) & bit) != 0u;
            }
        }
        count_wave(counts, kCheckSlot, bad);
        count_wave(counts, kCheckDuplicate, dup);
    }
}

// One workgroup per request. EXTEND (lens_b != nullptr): p = lens_a[b], e = lens_b[b],
// s = start[b]; the call reads positions 0 .. L - 1 with L = p + e (p for the ragged call).
// DECODE: L = lens_a[b] (positions past max_seq_len are never read: such a length is counted).
// page_shift > 0: table entries are pages of 2^page_shift slots.
__global__ __launch_bounds__(kChkThreads) void check_requests_kernel(
    const int32_t* __restrict__ table, int64_t table_rows, int64_t stride, int32_t page_shift,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ lens_a,
    const int32_t* __restrict__ lens_b, const int32_t* __restrict__ start, int64_t total,
    int32_t max_ext, int32_t max_seq, int64_t num_slots, bool ragged,
    const uint32_t* __restrict__ stored, int32_t* __restrict__ counts) {
    const int b = blockIdx.x;
    const bool ext = lens_b != nullptr;
    int64_t L;
    bool len_bad;
    bool reads;
    if (ext) {
        const int64_t p = lens_a[b], e = lens_b[b], s = start[b];
        len_bad = p < 0 || e < 0 || e > max_ext || p + e > max_seq || s < 0 || s + e > total;
        L = ragged ? p : p + e;
        reads = e > 0 && L > 0;  // a request with no suffix rows reads nothing
    } else {
        const int64_t l = lens_a[b];
        len_bad = l > max_seq;
        L = l;
        reads = l > 0;
    }
    const int64_t r = rpi[b];
    const bool row_bad = !len_bad && reads && (r < 0 || r >= table_rows);
    if (threadIdx.x == 0) {
        if (len_bad) atomicAdd(counts + kCheckLength, 1);
        if (row_bad) atomicAdd(counts + kCheckRow, 1);
    }
    if (len_bad || row_bad || !reads) return;  // uniform over the workgroup
    // L <= max_seq <= stride << page_shift (checked on the host): the row's entries suffice.
    const int32_t* row = table + r * stride;
    const int64_t P = (int64_t)1 << page_shift;
    for (int64_t j0 = 0; j0 < L; j0 += blockDim.x) {
        const int64_t j = j0 + threadIdx.x;
        bool bad = false, overlap = false;
        if (j < L) {
            const int64_t entry = row[j >> page_shift];
            bad = entry < 0 || (entry + 1) * P > num_slots;
            if (!bad && stored != nullptr) {
                const int64_t slot = entry * P + (j & (P - 1));
                overlap = ((stored[slot >> 5] >> (slot & 31)) & 1u) != 0u;
            }
        }
        count_wave(counts, kCheckSlot, bad);
        count_wave(counts, kCheckOverlap, overlap);
    }
}

int zero(void* p, int64_t words, hipStream_t stream) {
    if (words <= 0) return 0;
    const int64_t blocks = (words + kChkThreads - 1) / kChkThreads;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(kChkThreads), 0, stream, (uint32_t*)p, words);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mark(const int32_t* loc, int64_t n, int64_t num_slots, uint32_t* bitmap, int32_t* counts,
         hipStream_t stream) {
    if (zero(bitmap, check_bitmap_words(num_slots), stream)) return -1;
    if (n <= 0) return 0;
    const int64_t blocks = (n + kChkThreads - 1) / kChkThreads;
    hipLaunchKernelGGL(mark_slots_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(kChkThreads), 0, stream, loc, n, num_slots, bitmap, counts);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int64_t check_bitmap_words(int64_t num_slots) { return (num_slots + 31) / 32; }

int launch_check_store(const int32_t* loc, int64_t n, int64_t num_slots, void* bitmap,
                       int32_t* counts, hipStream_t stream) {
    if (zero(counts, kCheckCount, stream)) return -1;
    return mark(loc, n, num_slots, (uint32_t*)bitmap, counts, stream);
}

int launch_check_requests(const CheckArgs& c, hipStream_t stream) {
    if (zero(c.counts, kCheckCount, stream)) return -1;
    const uint32_t* stored = nullptr;
    if (c.store_loc != nullptr) {
        if (mark(c.store_loc, c.total, c.num_slots, (uint32_t*)c.bitmap, c.counts, stream)) return -1;
        stored = (const uint32_t*)c.bitmap;
    }
    if (c.batch <= 0) return 0;
    hipLaunchKernelGGL(check_requests_kernel, dim3((unsigned)c.batch), dim3(kChkThreads), 0, stream,
                       c.table, c.table_rows, c.stride, c.page_shift, c.rpi, c.lens_a, c.lens_b,
                       c.start, c.total, c.max_ext, c.max_seq, c.num_slots, c.ragged, stored,
                       c.counts);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace rax
