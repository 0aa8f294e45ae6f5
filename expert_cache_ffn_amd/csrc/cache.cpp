// The shared expert cache: host metadata of one LRU over (layer, expert) pairs,
// for all layers, in front of a fixed pool of device slots.
//
// techfeed summary of "Meet FreeToken" (MarkTechPost), section "Semantic-aware
// caching": during decode a single LRU expert cache spanning every MoE layer
// follows the router.  FreeToken paper explainer (ta-paperlens), section
// "Design: two-tier expert memory": a slot holds all tensors of one (layer,
// expert) pair, residency is decided on that logical pair, and since the host
// pool is the source of truth the cache can be rebuilt, shrunk or grown
// without changing any result.
//
// Policy readings where the pages are silent: hits are touched in the order
// given (ascending expert id from the forward call); a bind takes the lowest
// free slot, else the least recently used entry not used by the current
// layer-step; entries of the current layer-step are pinned until the next
// lookup opens a new one.  A whole-layer prefetch (explainer section "Prefill:
// full-layer double buffer and semantic anchors": the next layer streams into
// the same slot pool while the current one computes) holds its layer's
// entries until that layer's forward call; held entries are never evicted,
// and the experts a prefetch could not place stay reserved: a later prefetch
// leaves that many slots, so that forward call can still fill them on demand.
#include <memory>

#include "cache_internal.h"

using ecf::set_error;

namespace {
inline int64_t key_of(const ecf_cache *c, int32_t layer, int32_t e) { return (int64_t)layer * c->E + e; }

void unlink(ecf_cache *c, int32_t s)
{
    const int32_t p = c->prev[s], n = c->next[s];
    if (p >= 0)
        c->next[p] = n;
    else
        c->head = n;
    if (n >= 0)
        c->prev[n] = p;
    else
        c->tail = p;
    c->prev[s] = c->next[s] = -1;
}

void push_mru(ecf_cache *c, int32_t s)
{
    c->prev[s] = c->tail;
    c->next[s] = -1;
    if (c->tail >= 0)
        c->next[c->tail] = s;
    else
        c->head = s;
    c->tail = s;
}

bool pinned(const ecf_cache *c, int32_t s) { return c->pin_gen[s] == c->gen; }
bool evictable(const ecf_cache *c, int32_t s) { return !pinned(c, s) && !c->held[s]; }
}  // namespace

namespace ecf {

int32_t cache_available(const ecf_cache *c)
{
    int32_t blocked = c->n_pinned;  // resident slots no bind may take
    for (const auto &p : c->prefetched)
        for (int32_t s : p.slots)
            blocked += pinned(c, s) ? 0 : 1;
    return (int32_t)c->free.size() + (c->n_resident - blocked);
}

void cache_touch(ecf_cache *c, int32_t s)
{
    unlink(c, s);
    push_mru(c, s);
}

int32_t cache_bind(ecf_cache *c, int32_t layer, int32_t expert, int32_t *victim)
{
    int32_t s;
    *victim = -1;
    if (!c->free.empty()) {
        s = *c->free.begin();
        c->free.erase(c->free.begin());
    } else {
        s = c->head;
        while (s >= 0 && !evictable(c, s))
            s = c->next[s];
        if (s < 0)
            return -1;
        const int64_t old = c->key_of_slot[s];
        c->slot_of[old] = -1;
        unlink(c, s);
        --c->n_resident;
        *victim = (int32_t)old;
        ++c->stats.evictions;
    }
    const int64_t key = key_of(c, layer, expert);
    c->slot_of[key] = s;
    c->key_of_slot[s] = key;
    push_mru(c, s);
    ++c->n_resident;
    ++c->stats.inserts;
    return s;
}

hipEvent_t cache_take_prefetch(ecf_cache *c, int32_t layer)
{
    for (size_t i = 0; i < c->prefetched.size(); ++i) {
        auto &p = c->prefetched[i];
        if (p.layer != layer)
            continue;
        for (int32_t s : p.slots)
            c->held[s] = 0;
        c->reserve -= p.missing;
        hipEvent_t ev = p.done;
        c->prefetched.erase(c->prefetched.begin() + i);
        return ev;
    }
    return nullptr;
}

void cache_spare_event(ecf_cache *c, hipEvent_t ev)
{
    if (ev)
        c->spare_events.push_back(ev);
}

}  // namespace ecf

extern "C" {

int ecf_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t max_slots,
                     size_t slot_bytes, void *d_slots, const void *const *h_pool, int32_t host_threads,
                     ecf_cache **out)
{
    try {
        if (!out || n_layers <= 0 || n_experts <= 0 || n_slots < 0 || max_slots < n_slots ||
            (max_slots > 0 && (!d_slots || slot_bytes == 0)) || host_threads < 0)
            return set_error(ECF_EINVAL, "ecf_cache_create: bad arguments");
        std::unique_ptr<ecf_cache> c(new ecf_cache());  // freed if an allocation below throws
        c->L = n_layers;
        c->E = n_experts;
        c->n_slots = n_slots;
        c->max_slots = max_slots;
        c->slot_bytes = slot_bytes;
        c->d_slots = (char *)d_slots;
        if (h_pool)
            c->h_pool.assign(h_pool, h_pool + (size_t)n_layers * n_experts);
        c->slot_of.assign((size_t)n_layers * n_experts, -1);
        c->key_of_slot.assign(max_slots, -1);
        c->prev.assign(max_slots, -1);
        c->next.assign(max_slots, -1);
        c->pin_gen.assign(max_slots, 0);
        c->held.assign(max_slots, 0);
        for (int32_t s = 0; s < n_slots; ++s)
            c->free.insert(s);
        c->host_threads = host_threads;
        *out = c.release();
        return ECF_OK;
    } catch (...) {
        return set_error(ECF_EINVAL, "ecf_cache_create: allocation failed");
    }
}

void ecf_cache_destroy(ecf_cache *c)
{
    if (!c)
        return;
    ecf::cache_release_host(c);
    delete c;
}

int expert_cache_lookup(ecf_cache *c, int32_t layer, const int32_t *experts, int32_t n, int32_t *slots)
{
    return ::ecf::guarded("expert_cache_lookup", [&]() -> int {
        if (!c || layer < 0 || layer >= c->L || n < 0 || (n > 0 && (!experts || !slots)))
            return set_error(ECF_EINVAL, "expert_cache_lookup: bad arguments");
        for (int32_t i = 0; i < n; ++i)
            if (experts[i] < 0 || experts[i] >= c->E)
                return set_error(ECF_EINVAL, "expert_cache_lookup: expert %d out of range", experts[i]);
        ++c->gen;
        c->n_pinned = 0;
        c->step_layer = layer;
        for (int32_t i = 0; i < n; ++i) {
            const int32_t s = c->slot_of[key_of(c, layer, experts[i])];
            ++c->stats.lookups;
            slots[i] = s;
            if (s < 0) {
                ++c->stats.misses;
                continue;
            }
            ++c->stats.hits;
            ecf::cache_touch(c, s);
            if (!pinned(c, s)) {
                c->pin_gen[s] = c->gen;
                ++c->n_pinned;
            }
        }
        return ECF_OK;
    });
}

int32_t ecf_cache_available(const ecf_cache *c)
{
    if (!c)
        return set_error(ECF_EINVAL, "ecf_cache_available: NULL cache");
    return ecf::cache_available(c);
}

int expert_cache_evict(ecf_cache *c, int32_t layer, const int32_t *experts, int32_t n, int32_t *slots,
                       int32_t *victims)
{
    return ::ecf::guarded("expert_cache_evict", [&]() -> int {
        if (!c || n < 0 || (n > 0 && (!experts || !slots)))
            return set_error(ECF_EINVAL, "expert_cache_evict: bad arguments");
        if (c->step_layer < 0 || layer != c->step_layer)
            return set_error(ECF_ESTATE, "expert_cache_evict: layer %d has no open layer-step (lookup first)",
                             layer);
        for (int32_t i = 0; i < n; ++i) {
            if (experts[i] < 0 || experts[i] >= c->E)
                return set_error(ECF_EINVAL, "expert_cache_evict: expert %d out of range", experts[i]);
            if (c->slot_of[key_of(c, layer, experts[i])] >= 0)
                return set_error(ECF_EINVAL, "expert_cache_evict: expert %d already resident", experts[i]);
            for (int32_t j = 0; j < i; ++j)
                if (experts[j] == experts[i])
                    return set_error(ECF_EINVAL, "expert_cache_evict: expert %d repeated", experts[i]);
        }
        if (n > ecf_cache_available(c))
            return set_error(ECF_ENOSPC, "expert_cache_evict: %d slots wanted, %d available", n,
                             ecf_cache_available(c));
        for (int32_t i = 0; i < n; ++i) {
            int32_t victim = -1;
            const int32_t s = ecf::cache_bind(c, layer, experts[i], &victim);
            if (s < 0)  // cannot happen: availability was checked
                return set_error(ECF_ESTATE, "expert_cache_evict: no evictable slot");
            c->pin_gen[s] = c->gen;
            ++c->n_pinned;
            slots[i] = s;
            if (victims)
                victims[i] = victim;
        }
        return ECF_OK;
    });
}

int32_t ecf_cache_slot_of(const ecf_cache *c, int32_t layer, int32_t expert)
{
    if (!c || layer < 0 || layer >= c->L || expert < 0 || expert >= c->E)
        return set_error(ECF_EINVAL, "ecf_cache_slot_of: bad arguments");
    return c->slot_of[key_of(c, layer, expert)];
}

int ecf_cache_get_stats(const ecf_cache *c, ecf_cache_stats *out)
{
    return ::ecf::guarded("ecf_cache_get_stats", [&]() -> int {
        if (!c || !out)
            return set_error(ECF_EINVAL, "ecf_cache_get_stats: NULL argument");
        *out = c->stats;
        return ECF_OK;
    });
}

int ecf_cache_resize(ecf_cache *c, int32_t n_slots)
{
    return ::ecf::guarded("ecf_cache_resize", [&]() -> int {
        if (!c || n_slots < 0 || n_slots > c->max_slots)
            return set_error(ECF_EINVAL, "ecf_cache_resize: n_slots must be in [0, max_slots]");
        // a safe point: pending prefetch copies land first, and their holds end
        while (!c->prefetched.empty()) {
            hipEvent_t ev = ecf::cache_take_prefetch(c, c->prefetched.front().layer);
            if (ev && hipEventSynchronize(ev) != hipSuccess)
                return set_error(ECF_EHIP, "ecf_cache_resize: waiting for a prefetch failed");
            ecf::cache_spare_event(c, ev);
        }
        for (int32_t s = n_slots; s < c->n_slots; ++s) {
            c->free.erase(s);
            const int64_t key = c->key_of_slot[s];
            if (key >= 0) {
                c->slot_of[key] = -1;
                c->key_of_slot[s] = -1;
                unlink(c, s);
                --c->n_resident;
                if (pinned(c, s))
                    --c->n_pinned;
                c->pin_gen[s] = 0;
                ++c->stats.dropped;
            }
        }
        for (int32_t s = c->n_slots; s < n_slots; ++s)
            c->free.insert(s);
        c->n_slots = n_slots;
        c->step_layer = -1;  // a resize is a safe point: no layer-step stays open
        return ECF_OK;
    });
}

}  // extern "C"
