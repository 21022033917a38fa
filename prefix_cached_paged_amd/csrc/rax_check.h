// Internal (C++) interface of the debug checks of the device-side contracts (check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rax {

// Debug checks of the device-side contracts. The kinds of contract break they count, in the
// order of rax_check_item.
enum : int {
    kCheckLength = 0,
    kCheckRow = 1,
    kCheckSlot = 2,
    kCheckDuplicate = 3,
    kCheckOverlap = 4,
    kCheckCount = 5,
};

// Requests of one EXTEND (lens_b = extend_lens) or DECODE (lens_b = nullptr) call, validated on
// the host: max_seq <= stride << page_shift, and table holds table_rows rows of stride entries.
struct CheckArgs {
    const int32_t* table;
    int64_t table_rows;
    int64_t stride;
    int32_t page_shift;
    const int32_t* rpi;
    const int32_t* lens_a;  // prefix_lens (EXTEND) or seq_lens (DECODE)
    const int32_t* lens_b;  // extend_lens (EXTEND) or nullptr
    const int32_t* start;   // extend_start_loc (EXTEND) or nullptr
    int64_t total;          // total_extend_tokens: store_loc entries and the bound of start + e
    int32_t max_ext;
    int32_t max_seq;
    int64_t num_slots;
    bool ragged;
    const int32_t* store_loc;  // ragged store slots or nullptr
    void* bitmap;              // check_bitmap_words(num_slots) words when store_loc is given
    int32_t* counts;           // kCheckCount int32, zeroed by the launch
    int32_t batch;
};

int64_t check_bitmap_words(int64_t num_slots);
int launch_check_store(const int32_t* loc, int64_t n, int64_t num_slots, void* bitmap,
                       int32_t* counts, hipStream_t stream);
int launch_check_requests(const CheckArgs& c, hipStream_t stream);

}  // namespace rax
