// Controls of the fake device (fake_device.cpp).  Test infrastructure only.
#pragma once

#include <cstddef>
#include <cstdint>

namespace fake {
struct Counters {
    uint64_t host_mallocs = 0;      // pinned staging buffers allocated
    uint64_t copies = 0;            // host-to-device copies enqueued
    uint64_t queries = 0;           // event queries
    uint64_t launches = 0;          // kernel launches enqueued
    uint64_t launches_checked = 0;  // launches run that found their own tables
    uint64_t tables_checked = 0;    // launches whose tables passed check_tables
};
void run(size_t n);        // run the next n queued operations, in order
void run_all();
size_t queued();
void allow_wait(bool allow);  // let hipEventSynchronize run the queue (release only)
const Counters& counts();
size_t pinned_live();
}  // namespace fake
