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
    // Whole-layer prefetches not yet consumed by that layer's forward call:
    // their resident entries are held (no bind evicts them) and `missing` of
    // the layer's experts did not fit; `reserve` (the sum of those) is what
    // a later prefetch leaves for those forward calls to fill on demand.
    struct Prefetch {
        int32_t layer = -1, missing = 0;
        std::vector<int32_t> slots;    // held slots
        hipEvent_t done = nullptr;     // recorded on the copy stream after the layer's copies
    };
    std::vector<Prefetch> prefetched;
    std::vector<char> held;            // [max_slots] 1 while held by a prefetch
    int32_t reserve = 0;
    std::vector<hipEvent_t> spare_events;
    hipEvent_t last_compute = nullptr; // recorded after each cache-mode forward's kernels
    bool have_last_compute = false;
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
// Slots a bind could take now: free ones plus resident entries neither pinned
// by the open layer-step nor held by a prefetch.
int32_t cache_available(const ecf_cache *c);
// Bind (layer, expert) to the lowest free slot, else to the least recently used
// evictable entry (evicted; its key -> *victim, else -1).  Becomes MRU.  The
// caller has checked availability.  Returns the slot, or -1 if none.
int32_t cache_bind(ecf_cache *c, int32_t layer, int32_t expert, int32_t *victim);
// Move a resident slot to the most recently used end.
void cache_touch(ecf_cache *c, int32_t slot);
// End the hold of `layer`'s pending prefetch (if any): returns its copy event
// (the caller's compute stream must wait on it before reading the layer's
// slots, then give it back with cache_spare_event) or nullptr.
hipEvent_t cache_take_prefetch(ecf_cache *c, int32_t layer);
void cache_spare_event(ecf_cache *c, hipEvent_t ev);
// Grow a pinned host staging buffer to at least `bytes` (hipHostMalloc).
int staging(ecf_cache::Staging &s, size_t bytes);
void cache_release_host(ecf_cache *c);
}  // namespace ecf
