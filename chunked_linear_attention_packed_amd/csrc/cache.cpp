// Host directory of a device-resident view-state cache.
//
// Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "Long
// Requests": branches of one request are split into shards that each need the
// full view; GPU nodes keep the linear-attention state of recent views so a
// shard does not recompute its view, and shards are routed to the node that
// holds their view.  The states live in a caller-owned device pool
// [capacity][H][d_k][d_v] (usable directly as the ext_state of a pass); this
// directory maps view ids to pool rows and evicts the least recently used
// row when a new view needs one.
#include <cstdint>
#include <list>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "linattn.h"

struct la_state_cache {
    int32_t capacity = 0;
    // most recently used at the front: (view id, row)
    std::list<std::pair<int64_t, int32_t>> lru;
    std::unordered_map<int64_t, std::list<std::pair<int64_t, int32_t>>::iterator> where;
    std::vector<int32_t> free_rows;   // rows never used or erased, taken from the back
};

extern "C" la_status la_cache_create(int32_t capacity, la_state_cache** cache) {
    if (!cache || capacity < 1 || capacity > (1 << 30)) return LA_ERR_INVALID_ARG;
    la_state_cache* c = new (std::nothrow) la_state_cache;
    if (!c) return LA_ERR_INVALID_ARG;
    c->capacity = capacity;
    c->free_rows.reserve(size_t(capacity));
    for (int32_t r = capacity - 1; r >= 0; --r) c->free_rows.push_back(r);   // row 0 first
    *cache = c;
    return LA_OK;
}

extern "C" la_status la_cache_destroy(la_state_cache* cache) {
    if (!cache) return LA_ERR_INVALID_ARG;
    delete cache;
    return LA_OK;
}

extern "C" la_status la_cache_lookup(la_state_cache* cache, int64_t view_id, int32_t* row) {
    if (!cache || !row || view_id < 0) return LA_ERR_INVALID_ARG;
    auto it = cache->where.find(view_id);
    if (it == cache->where.end()) {
        *row = -1;
        return LA_OK;
    }
    cache->lru.splice(cache->lru.begin(), cache->lru, it->second);   // now most recent
    *row = it->second->second;
    return LA_OK;
}

extern "C" la_status la_cache_reserve(la_state_cache* cache, int64_t view_id, int32_t* row,
                                      int64_t* evicted_id) {
    if (!cache || !row || view_id < 0) return LA_ERR_INVALID_ARG;
    int64_t evicted = -1;
    auto it = cache->where.find(view_id);
    if (it != cache->where.end()) {
        cache->lru.splice(cache->lru.begin(), cache->lru, it->second);
        *row = it->second->second;
    } else {
        int32_t r;
        if (!cache->free_rows.empty()) {
            r = cache->free_rows.back();
            cache->free_rows.pop_back();
        } else {
            // evict the least recently used view and reuse its row
            const auto victim = cache->lru.back();
            evicted = victim.first;
            r = victim.second;
            cache->where.erase(victim.first);
            cache->lru.pop_back();
        }
        cache->lru.emplace_front(view_id, r);
        cache->where[view_id] = cache->lru.begin();
        *row = r;
    }
    if (evicted_id) *evicted_id = evicted;
    return LA_OK;
}

extern "C" la_status la_cache_erase(la_state_cache* cache, int64_t view_id) {
    if (!cache || view_id < 0) return LA_ERR_INVALID_ARG;
    auto it = cache->where.find(view_id);
    if (it == cache->where.end()) return LA_OK;
    cache->free_rows.push_back(it->second->second);
    cache->lru.erase(it->second);
    cache->where.erase(it);
    return LA_OK;
}

extern "C" la_status la_cache_count(const la_state_cache* cache, int32_t* n) {
    if (!cache || !n) return LA_ERR_INVALID_ARG;
    *n = int32_t(cache->where.size());
    return LA_OK;
}
