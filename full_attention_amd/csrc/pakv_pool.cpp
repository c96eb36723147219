// Page pools: which physical pages a sequence holds, per group of layers, and
// how many tokens a byte budget buys.
//
// The two attention groups want different page lifetimes (pegainfer issue
// #807, Description, first paragraph: the sliding group releases pages the
// full group still reads): a full layer may read any position of a sequence,
// a sliding layer only its last W.  So each group gets its own pool and page
// table, and a window pool hands a sequence's pages back once every query that
// can still come lies W or more positions past them.  FreeToken PR #898 sizes
// the window pool beside the full one ("End to end": the bracketed window
// pool, one token for every five of the full pool in each printed row).
//
// Host bookkeeping only: the table is host memory the caller copies to the
// device before the calls that read it.

#include <cstring>
#include <new>
#include <vector>

#include "pakv_internal.h"

struct pakv_page_pool {
    int32_t num_pages;
    int32_t max_seqs;
    int32_t max_pages_per_seq;
    int32_t window;
    std::vector<int32_t> table;      // [max_seqs][max_pages_per_seq], -1 where nothing is held
    std::vector<int32_t> free_list;  // a stack: the last page released is the next handed out
    std::vector<int32_t> released;   // pages released by the last reserve / release_seq
};

using namespace pakv;

extern "C" {

pakv_status pakv_page_pool_create(int32_t num_pages, int32_t max_seqs, int32_t max_pages_per_seq, int32_t window,
                                  pakv_page_pool** out) {
    clear_error();
    if (!out) return fail(PAKV_ERR_INVALID, "out is null");
    *out = nullptr;
    if (num_pages <= 0 || max_seqs <= 0 || max_pages_per_seq <= 0 || window < 0)
        return fail(PAKV_ERR_INVALID, "pool sizes must be positive and the window not negative");
    pakv_page_pool* p = new (std::nothrow) pakv_page_pool;
    if (!p) return fail(PAKV_ERR_INVALID, "out of host memory");
    p->num_pages = num_pages;
    p->max_seqs = max_seqs;
    p->max_pages_per_seq = max_pages_per_seq;
    p->window = window;
    p->table.assign((size_t)max_seqs * max_pages_per_seq, -1);
    p->free_list.resize(num_pages);
    for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;   // page 0 handed out first
    *out = p;
    return PAKV_OK;
}

void pakv_page_pool_destroy(pakv_page_pool* pool) { delete pool; }

pakv_status pakv_page_pool_reserve(pakv_page_pool* pool, int32_t seq, int32_t first_query, int32_t end) {
    clear_error();
    if (!pool) return fail(PAKV_ERR_INVALID, "pool is null");
    if (seq < 0 || seq >= pool->max_seqs) return fail(PAKV_ERR_INVALID, "sequence %d out of range", seq);
    if (first_query < 0 || end < 0 || first_query > end)
        return fail(PAKV_ERR_INVALID, "need 0 <= first_query <= end (%d, %d)", first_query, end);
    if ((int64_t)end > (int64_t)pool->max_pages_per_seq * PAKV_PAGE_SIZE)
        return fail(PAKV_ERR_INVALID, "end %d past the table's %d positions", end,
                    pool->max_pages_per_seq * PAKV_PAGE_SIZE);
    int32_t* row = pool->table.data() + (size_t)seq * pool->max_pages_per_seq;
    // keys a query at first_query or later can see start at first_query - W + 1
    const int32_t keep_from = pool->window > 0 ? (first_query - pool->window + 1 > 0 ? first_query - pool->window + 1 : 0)
                                               : 0;
    const int32_t page_lo = keep_from / PAKV_PAGE_SIZE;
    const int32_t page_hi = (end + PAKV_PAGE_SIZE - 1) / PAKV_PAGE_SIZE;
    // pages needed that are not held yet; refuse before changing anything
    int32_t need = 0, freed = 0;
    for (int32_t i = page_lo; i < page_hi; ++i) need += row[i] < 0;
    for (int32_t i = 0; i < page_lo; ++i) freed += row[i] >= 0;
    if (need > (int32_t)pool->free_list.size() + freed)
        return fail(PAKV_ERR_WORKSPACE, "page pool exhausted: %d pages needed, %d free", need,
                    (int32_t)pool->free_list.size() + freed);
    pool->released.clear();
    for (int32_t i = 0; i < page_lo; ++i) {
        if (row[i] >= 0) {
            pool->released.push_back(row[i]);
            pool->free_list.push_back(row[i]);
            row[i] = -1;
        }
    }
    for (int32_t i = page_lo; i < page_hi; ++i) {
        if (row[i] < 0) {
            row[i] = pool->free_list.back();
            pool->free_list.pop_back();
        }
    }
    return PAKV_OK;
}

pakv_status pakv_page_pool_release_seq(pakv_page_pool* pool, int32_t seq) {
    clear_error();
    if (!pool) return fail(PAKV_ERR_INVALID, "pool is null");
    if (seq < 0 || seq >= pool->max_seqs) return fail(PAKV_ERR_INVALID, "sequence %d out of range", seq);
    int32_t* row = pool->table.data() + (size_t)seq * pool->max_pages_per_seq;
    pool->released.clear();
    for (int32_t i = 0; i < pool->max_pages_per_seq; ++i) {
        if (row[i] >= 0) {
            pool->released.push_back(row[i]);
            pool->free_list.push_back(row[i]);
            row[i] = -1;
        }
    }
    return PAKV_OK;
}

const int32_t* pakv_page_pool_table(const pakv_page_pool* pool) { return pool ? pool->table.data() : nullptr; }

int32_t pakv_page_pool_free_pages(const pakv_page_pool* pool) { return pool ? (int32_t)pool->free_list.size() : -1; }

int32_t pakv_page_pool_released(const pakv_page_pool* pool, int32_t* out, int32_t cap) {
    if (!pool) return -1;
    const int32_t n = (int32_t)pool->released.size();
    if (out)
        for (int32_t i = 0; i < n && i < cap; ++i) out[i] = pool->released[i];
    return n;
}

pakv_status pakv_pool_tokens(const pakv_layer_map* map, int64_t budget_bytes, double window_share,
                             int64_t* full_tokens, int64_t* window_tokens) {
    clear_error();
    if (!map || !full_tokens || !window_tokens) return fail(PAKV_ERR_INVALID, "null pointer");
    if (budget_bytes < 0 || !(window_share >= 0.0) || window_share > 1e9)
        return fail(PAKV_ERR_INVALID, "budget must not be negative and the share finite and not negative");
    int64_t fb = 0, wb = 0;
    if (pakv_status s = pakv_kv_bytes_per_token(map, &fb, &wb)) return s;
    const double per = (double)fb + window_share * (double)wb;
    if (!(per > 0.0)) return fail(PAKV_ERR_INVALID, "the map stores no bytes per token");
    const int64_t full = (int64_t)((double)budget_bytes / per);
    *full_tokens = full;
    *window_tokens = (int64_t)(window_share * (double)full);
    return PAKV_OK;
}

}  // extern "C"
