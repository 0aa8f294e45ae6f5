// Definition of ecf_cache (opaque in the ABI) and the host-side helpers the
// forward call uses with it.
#pragma once

#include <set>
#include <vector>

#include "ecf_internal.h"
#include "host_ffn.h"

struct ecf_cache {
    int32_t L = 0, E = 0, n_slots = 0, max_slots = 0;
    size_t slot_bytes = 0;
    char *d_slots = nullptr;
    std::vector<const void *> h_pool;  // [L * E] pinned host blobs (source of truth)
    std::vector<int32_t> slot_of;      // [L * E] -> slot or -1
    std::vector<int64_t> key_of_slot;  // [max_slots] -> layer * E + expert or -1
    std::vector<int32_t> prev, next;   // LRU list over slots: head = least recent
    int32_t head = -1, tail = -1;
    std::set<int32_t> free;            // free slot ids, lowest first
    std::vector<uint32_t> pin_gen;     // slot pinned iff pin_gen == gen
    uint32_t gen = 1;
    int32_t n_resident = 0, n_pinned = 0;
    int32_t step_layer = -1;           // layer of the open layer-step, -1 if none
    ecf_cache_stats stats{};
    int32_t host_threads = 0;
    // forward-call host resources, created on first use
    ecf::HostPool *pool = nullptr;
    struct Staging {
        void *p = nullptr;
        size_t bytes = 0;
    } st_counts, st_idx, st_gate, st_x, st_out, st_ptrs, st_y;
    hipEvent_t copy_done = nullptr;
};

namespace ecf {
// Grow a pinned host staging buffer to at least `bytes` (hipHostMalloc).
int staging(ecf_cache::Staging &s, size_t bytes);
void cache_release_host(ecf_cache *c);
}  // namespace ecf
