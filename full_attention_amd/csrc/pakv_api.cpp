// C ABI of the paged KV-cache attention library: argument checks, the layer
// map (ownership and KV-source aliasing), the decode split plan and dispatch to
// the kernel launchers.  Nothing here touches the GPU before every argument has
// been checked.

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "pakv_internal.h"

namespace pakv {

static thread_local std::string g_last_error;

struct TimingHook {
    void* const* events = nullptr;
    int32_t pairs = 0;
    int32_t used = 0;
    int32_t mask = 0;
};
static thread_local TimingHook g_timing;
static std::atomic<int32_t> g_decode_checks{0};

int32_t decode_checks() { return g_decode_checks.load(std::memory_order_relaxed); }

pakv_status fail(pakv_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

int timing_slot(int kind) {
    if (!g_timing.events || !(g_timing.mask & kind) || g_timing.used >= g_timing.pairs) return -1;
    return g_timing.used++;
}

void* const* timing_events() { return g_timing.events; }

TimingPause::TimingPause()
    : events(g_timing.events), pairs(g_timing.pairs), used(g_timing.used), mask(g_timing.mask) {
    g_timing.events = nullptr;
    g_timing.pairs = 0;
}

TimingPause::~TimingPause() {
    g_timing.events = events;
    g_timing.pairs = pairs;
    g_timing.used = used;
    g_timing.mask = mask;
}

DecodePlan plan_decode(const pakv_layer_desc& d, int32_t num_seqs) {
    DecodePlan p{};
    p.grid = kDecodeGrid;
    p.units = num_seqs * d.num_kv_heads;
    p.group = d.num_q_heads / d.num_kv_heads;
    return p;
}

// Workspace: the status word's block, arrival counters (a fixed region of
// kDecodeMaxUnits, so that layers of any shape can share one workspace and
// leave it zeroed), then partial o, then partial (m, l); 256-byte aligned
// parts.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_partial_bytes(const pakv_layer_desc& d, int32_t num_seqs) {
    DecodePlan p = plan_decode(d, num_seqs);
    size_t slots = (size_t)(p.grid + p.units) * p.group;
    return kDecodeStatusBytes + align256((size_t)kDecodeMaxUnits * sizeof(uint32_t)) +
           align256(slots * d.head_dim * sizeof(float)) + align256(slots * 2 * sizeof(float));
}

PlanLayout plan_layout(int32_t num_seqs, int32_t hkv, int32_t max_kv_len) {
    PlanLayout l;
    l.soff = kPlanHeader;
    l.slen = l.soff + num_seqs + 1;
    l.rec = (l.slen + num_seqs + 15) & ~(int64_t)15;
    l.ids = l.rec + (int64_t)kDecodeGrid * kPlanRecord;
    l.cap = (int64_t)num_seqs * hkv * ((max_kv_len + 15) / 16);
    l.words = l.ids + l.cap;
    return l;
}

size_t decode_plan_bytes(const pakv_layer_desc& d, int32_t num_seqs, int32_t max_kv_len) {
    return align256((size_t)plan_layout(num_seqs, d.num_kv_heads, max_kv_len).words * sizeof(int32_t));
}

size_t decode_workspace_bytes(const pakv_layer_desc& d, int32_t num_seqs, int32_t max_kv_len) {
    return decode_partial_bytes(d, num_seqs) + decode_plan_bytes(d, num_seqs, max_kv_len);
}

static bool layer_ok(const pakv_layer_map* m, int32_t layer) {
    return m && layer >= 0 && layer < (int32_t)m->layers.size();
}

}  // namespace pakv

using namespace pakv;

extern "C" {

const char* pakv_last_error(void) { return g_last_error.c_str(); }

pakv_status pakv_set_timing_events(void* const* events, int32_t n_pairs, int32_t kernel_mask) {
    clear_error();
    if (events && n_pairs < 0) return fail(PAKV_ERR_INVALID, "n_pairs < 0");
    g_timing.events = events;
    g_timing.pairs = events ? n_pairs : 0;
    g_timing.used = 0;
    g_timing.mask = kernel_mask;
    return PAKV_OK;
}

int32_t pakv_timing_pairs_used(void) { return g_timing.used; }

pakv_status pakv_set_decode_checks(int32_t flags) {
    clear_error();
    if (flags & ~(int32_t)PAKV_CHECK_XCD_PLACEMENT) return fail(PAKV_ERR_INVALID, "unknown check flags 0x%x", flags);
    g_decode_checks.store(flags, std::memory_order_relaxed);
    return PAKV_OK;
}

pakv_status pakv_resolve_kv_sources(int32_t n_layers, const int32_t* layer_type,
                                    int32_t first_shared, int32_t* out_source) {
    clear_error();
    if (n_layers < 0) return fail(PAKV_ERR_INVALID, "n_layers < 0");
    if (n_layers > 0 && (!layer_type || !out_source)) return fail(PAKV_ERR_INVALID, "null pointer");
    if (first_shared < 0) return fail(PAKV_ERR_INVALID, "first_shared < 0");
    std::vector<int32_t> src(n_layers);
    for (int32_t l = 0; l < n_layers; ++l) {
        if (l < first_shared) { src[l] = l; continue; }
        int32_t found = -1;
        for (int32_t i = first_shared - 1; i >= 0; --i) {
            if (i < n_layers && layer_type[i] == layer_type[l]) { found = i; break; }
        }
        if (found < 0)
            return fail(PAKV_ERR_ALIAS, "KV-shared layer %d has no earlier layer of its type (%d)",
                        l, layer_type[l]);
        src[l] = found;
    }
    for (int32_t l = 0; l < n_layers; ++l) out_source[l] = src[l];
    return PAKV_OK;
}

pakv_status pakv_layer_map_create(const pakv_layer_desc* descs, int32_t n, pakv_layer_map** out) {
    clear_error();
    if (!out) return fail(PAKV_ERR_INVALID, "out is null");
    *out = nullptr;
    if (n <= 0) return fail(PAKV_ERR_INVALID, "a layer map needs at least one layer");
    if (!descs) return fail(PAKV_ERR_INVALID, "descs is null");
    for (int32_t l = 0; l < n; ++l) {
        const pakv_layer_desc& d = descs[l];
        if (d.head_dim != 256 && d.head_dim != 512)
            return fail(PAKV_ERR_UNSUPPORTED, "layer %d: head_dim %d (256 or 512 supported)", l, d.head_dim);
        if (d.num_kv_heads < 1 || d.num_q_heads < 1)
            return fail(PAKV_ERR_INVALID, "layer %d: head counts must be positive", l);
        if (d.num_q_heads % d.num_kv_heads != 0)
            return fail(PAKV_ERR_INVALID, "layer %d: Hq %d is not a multiple of Hkv %d", l,
                        d.num_q_heads, d.num_kv_heads);
        if (d.num_q_heads / d.num_kv_heads > 16)
            return fail(PAKV_ERR_UNSUPPORTED, "layer %d: group size %d above 16", l,
                        d.num_q_heads / d.num_kv_heads);
        if (d.window < 0) return fail(PAKV_ERR_INVALID, "layer %d: negative window", l);
        if (d.kv_dtype != PAKV_KV_BF16 && d.kv_dtype != PAKV_KV_INT8_PTH && d.kv_dtype != PAKV_KV_FP8_PTH)
            return fail(PAKV_ERR_INVALID, "layer %d: unknown kv_dtype %d", l, d.kv_dtype);
        if (d.k_eq_v != 0 && d.k_eq_v != 1) return fail(PAKV_ERR_INVALID, "layer %d: k_eq_v must be 0 or 1", l);
        if (d.k_eq_v && !(d.v_norm_eps >= 0.0f && d.v_norm_eps < 1e30f))
            return fail(PAKV_ERR_INVALID, "layer %d: v_norm_eps must be finite and not negative", l);
        if (d.k_eq_v && d.kv_dtype != PAKV_KV_BF16)
            return fail(PAKV_ERR_UNSUPPORTED, "layer %d: K=V storage is built for bf16 layers only", l);
        if (!(d.sm_scale > 0.0f) || d.sm_scale != d.sm_scale || d.sm_scale > 1e30f)
            return fail(PAKV_ERR_INVALID, "layer %d: sm_scale must be positive and finite", l);
        if (d.kv_source != -1) {
            int32_t s = d.kv_source;
            if (s < 0 || s >= l)
                return fail(PAKV_ERR_ALIAS, "layer %d: kv_source %d is not an earlier layer", l, s);
            const pakv_layer_desc& sd = descs[s];
            if (sd.kv_source != -1)
                return fail(PAKV_ERR_ALIAS, "layer %d: kv_source %d is itself KV-shared", l, s);
            if (sd.head_dim != d.head_dim || sd.num_kv_heads != d.num_kv_heads ||
                sd.window != d.window || sd.kv_dtype != d.kv_dtype || sd.k_eq_v != d.k_eq_v ||
                (d.k_eq_v && sd.v_norm_eps != d.v_norm_eps))
                return fail(PAKV_ERR_ALIAS,
                            "layer %d: kv_source %d differs in head_dim, num_kv_heads, window, kv_dtype or "
                            "K=V storage", l, s);
        }
    }
    pakv_layer_map* m = new (std::nothrow) pakv_layer_map;
    if (!m) return fail(PAKV_ERR_INVALID, "out of host memory");
    m->layers.resize(n);
    for (int32_t l = 0; l < n; ++l) {
        m->layers[l].desc = descs[l];
        m->layers[l].source = descs[l].kv_source == -1 ? l : descs[l].kv_source;
        m->layers[l].bound = false;
        std::memset(&m->layers[l].slab, 0, sizeof(pakv_slab));
    }
    *out = m;
    // a PAKV_DEBUG_BOUNDS build takes its counters' device address here,
    // before any call that a caller may capture into a graph
    (void)debug_bad_ids_ptr();
    return PAKV_OK;
}

void pakv_layer_map_destroy(pakv_layer_map* map) { delete map; }

static pakv_status hip_status(int err, const char* what);

pakv_status pakv_debug_bounds_counts(uint32_t* counts) {
    clear_error();
#ifdef PAKV_DEBUG_BOUNDS
    if (!counts) return fail(PAKV_ERR_INVALID, "counts is null");
    return hip_status(debug_bad_ids_read(counts, PAKV_DEBUG_COUNTS), "debug_bounds_counts");
#else
    (void)counts;
    return fail(PAKV_ERR_UNSUPPORTED, "page ids are counted only by a PAKV_DEBUG_BOUNDS build");
#endif
}

pakv_status pakv_debug_bounds_reset(void) {
    clear_error();
#ifdef PAKV_DEBUG_BOUNDS
    return hip_status(debug_bad_ids_reset(), "debug_bounds_reset");
#else
    return fail(PAKV_ERR_UNSUPPORTED, "page ids are counted only by a PAKV_DEBUG_BOUNDS build");
#endif
}

pakv_status pakv_layer_map_bind_slab(pakv_layer_map* map, int32_t layer, const pakv_slab* slab) {
    clear_error();
    if (!layer_ok(map, layer)) return fail(PAKV_ERR_INVALID, "bad map or layer %d", layer);
    if (!slab) return fail(PAKV_ERR_INVALID, "slab is null");
    auto& L = map->layers[layer];
    if (L.source != layer)
        return fail(PAKV_ERR_ALIAS, "layer %d is KV-shared (reads layer %d) and owns no slab", layer, L.source);
    if (slab->page_size != PAKV_PAGE_SIZE)
        return fail(PAKV_ERR_UNSUPPORTED, "page_size %d (16 supported)", slab->page_size);
    if (slab->num_pages <= 0) return fail(PAKV_ERR_INVALID, "num_pages must be positive");
    if (!slab->k || (!slab->v && !L.desc.k_eq_v)) return fail(PAKV_ERR_INVALID, "slab k or v is null");
    if (L.desc.kv_dtype != PAKV_KV_BF16 && (!slab->k_scale || !slab->v_scale))
        return fail(PAKV_ERR_INVALID, "an 8-bit slab needs k_scale and v_scale");
    L.slab = *slab;
    L.bound = true;
    return PAKV_OK;
}

pakv_status pakv_layer_map_source(const pakv_layer_map* map, int32_t layer, int32_t* src) {
    clear_error();
    if (!layer_ok(map, layer) || !src) return fail(PAKV_ERR_INVALID, "bad map, layer or src");
    *src = map->layers[layer].source;
    return PAKV_OK;
}

pakv_status pakv_kv_bytes_per_token(const pakv_layer_map* map, int64_t* full_bytes, int64_t* window_bytes) {
    clear_error();
    if (!map || !full_bytes || !window_bytes) return fail(PAKV_ERR_INVALID, "null pointer");
    int64_t f = 0, w = 0;
    for (size_t l = 0; l < map->layers.size(); ++l) {
        const auto& L = map->layers[l];
        if (L.source != (int32_t)l) continue;
        const pakv_layer_desc& d = L.desc;
        int64_t row = d.kv_dtype == PAKV_KV_BF16 ? 2 * (int64_t)d.head_dim : (int64_t)d.head_dim + 4;
        int64_t bytes = (int64_t)d.num_kv_heads * (d.k_eq_v ? 1 : 2) * row;
        if (d.window == 0) f += bytes; else w += bytes;
    }
    *full_bytes = f;
    *window_bytes = w;
    return PAKV_OK;
}

pakv_status pakv_slab_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_pages,
                            size_t* code_bytes, size_t* scale_bytes) {
    clear_error();
    if (!layer_ok(map, layer) || !code_bytes || !scale_bytes) return fail(PAKV_ERR_INVALID, "bad arguments");
    if (num_pages < 0) return fail(PAKV_ERR_INVALID, "num_pages < 0");
    const pakv_layer_desc& d = map->layers[layer].desc;
    size_t rows = (size_t)num_pages * d.num_kv_heads * PAKV_PAGE_SIZE;
    *code_bytes = rows * d.head_dim * (d.kv_dtype == PAKV_KV_BF16 ? 2 : 1);
    *scale_bytes = d.kv_dtype == PAKV_KV_BF16 ? 0 : rows * sizeof(float);
    return PAKV_OK;
}

static pakv_status check_pages(const pakv_pages* pages, int32_t num_seqs) {
    if (!pages || !pages->page_table) return fail(PAKV_ERR_INVALID, "pages or page_table is null");
    if (pages->max_pages_per_seq <= 0) return fail(PAKV_ERR_INVALID, "max_pages_per_seq must be positive");
    if (pages->num_seqs < num_seqs)
        return fail(PAKV_ERR_INVALID, "page table has %d sequences, call needs %d", pages->num_seqs, num_seqs);
    return PAKV_OK;
}

static SlabView view_of(const pakv_layer_map::Layer& src) {
    SlabView s;
    s.k = src.slab.k;
    s.v = src.slab.v;
    s.k_scale = src.slab.k_scale;
    s.v_scale = src.slab.v_scale;
    s.num_pages = src.slab.num_pages;
    return s;
}

static pakv_status hip_status(int err, const char* what) {
    if (err == 0) return PAKV_OK;
    return fail(PAKV_ERR_HIP, "%s: %s", what, hip_error_string(err));
}

pakv_status pakv_paged_kv_store(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                const int32_t* cu_tokens, const int32_t* start_pos,
                                const void* k, const void* v,
                                int32_t num_seqs, int32_t total_tokens, void* stream) {
    clear_error();
    if (!layer_ok(map, layer)) return fail(PAKV_ERR_INVALID, "bad map or layer %d", layer);
    const auto& L = map->layers[layer];
    if (L.source != layer) return PAKV_OK;   // shared layer: the source already stored these rows
    if (num_seqs < 0 || total_tokens < 0) return fail(PAKV_ERR_INVALID, "negative sizes");
    if (pakv_status s = check_pages(pages, num_seqs)) return s;
    if (!cu_tokens || !start_pos) return fail(PAKV_ERR_INVALID, "cu_tokens or start_pos is null");
    if (total_tokens > 0 && (!k || (!v && !L.desc.k_eq_v))) return fail(PAKV_ERR_INVALID, "k or v is null");
    if (!L.bound) return fail(PAKV_ERR_INVALID, "layer %d has no slab bound", layer);
    if (total_tokens == 0 || num_seqs == 0) return PAKV_OK;
    StoreLaunch a;
    a.slab = view_of(L);
    a.page_table = pages->page_table;
    a.max_pages = pages->max_pages_per_seq;
    a.cu_tokens = cu_tokens;
    a.start_pos = start_pos;
    a.k = static_cast<const uint16_t*>(k);
    a.v = L.desc.k_eq_v ? nullptr : static_cast<const uint16_t*>(v);
    a.num_seqs = num_seqs;
    a.total_tokens = total_tokens;
    a.hkv = L.desc.num_kv_heads;
    a.head_dim = L.desc.head_dim;
    a.kv_dtype = L.desc.kv_dtype;
    return hip_status(launch_store(a, stream), "paged_kv_store launch");
}

size_t pakv_decode_workspace_bytes(const pakv_layer_map* map, int32_t layer,
                                   int32_t num_seqs, int32_t max_kv_len) {
    if (!layer_ok(map, layer) || num_seqs < 0 || max_kv_len < 1) return 0;
    return decode_workspace_bytes(map->layers[layer].desc, num_seqs, max_kv_len);
}

size_t pakv_decode_plan_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_seqs, int32_t max_kv_len) {
    if (!layer_ok(map, layer) || num_seqs < 0 || max_kv_len < 1) return 0;
    return decode_plan_bytes(map->layers[layer].desc, num_seqs, max_kv_len);
}

// Checks shared by the decode calls and fills everything but the buffers.
static pakv_status decode_setup(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                int32_t num_seqs, int32_t max_kv_len, DecodeLaunch& a) {
    if (!layer_ok(map, layer)) return fail(PAKV_ERR_INVALID, "bad map or layer %d", layer);
    if (num_seqs < 0) return fail(PAKV_ERR_INVALID, "num_seqs < 0");
    if (max_kv_len < 1) return fail(PAKV_ERR_INVALID, "max_kv_len must be at least 1");
    if (num_seqs == 0) return PAKV_OK;
    if (pakv_status s = check_pages(pages, num_seqs)) return s;
    if ((int64_t)max_kv_len > (int64_t)pages->max_pages_per_seq * PAKV_PAGE_SIZE)
        return fail(PAKV_ERR_INVALID, "max_kv_len %d exceeds the page table's %d positions", max_kv_len,
                    pages->max_pages_per_seq * PAKV_PAGE_SIZE);
    const auto& L = map->layers[layer];
    const auto& S = map->layers[L.source];
    if (!S.bound) return fail(PAKV_ERR_INVALID, "slab of layer %d (source of %d) is not bound", L.source, layer);
    if (num_seqs > kDecodeMaxSeqs)
        return fail(PAKV_ERR_UNSUPPORTED, "num_seqs %d above %d per decode call", num_seqs, kDecodeMaxSeqs);
    if ((int64_t)num_seqs * L.desc.num_kv_heads > kDecodeMaxUnits)
        return fail(PAKV_ERR_UNSUPPORTED, "num_seqs * Hkv = %lld above %d per decode call",
                    (long long)num_seqs * L.desc.num_kv_heads, kDecodeMaxUnits);
    a = DecodeLaunch{};
    a.slab = view_of(S);
    a.page_table = pages->page_table;
    a.max_pages = pages->max_pages_per_seq;
    a.num_seqs = num_seqs;
    a.max_kv_len = max_kv_len;
    a.hq = L.desc.num_q_heads;
    a.hkv = L.desc.num_kv_heads;
    a.head_dim = L.desc.head_dim;
    a.window = L.desc.window;
    a.kv_dtype = L.desc.kv_dtype;
    a.k_eq_v = S.desc.k_eq_v;
    a.v_norm_eps = S.desc.v_norm_eps;
    a.sm_scale = L.desc.sm_scale;
    a.check_xcd = (decode_checks() & PAKV_CHECK_XCD_PLACEMENT) ? 1 : 0;
    a.plan = plan_decode(L.desc, num_seqs);
    a.layout = plan_layout(num_seqs, a.hkv, max_kv_len);
    return PAKV_OK;
}

// Workspace: the status word (in a block of kDecodeStatusBytes), arrival
// counters (a fixed region of kDecodeMaxUnits, so that layers of any shape
// can share one workspace and leave it zeroed), partial o, partial (m, l);
// then, for the unplanned call, its schedule.
static void bind_partials(DecodeLaunch& a, void* workspace) {
    size_t slots = (size_t)(a.plan.grid + a.plan.units) * a.plan.group;
    char* ws = static_cast<char*>(workspace);
    a.status = reinterpret_cast<uint32_t*>(ws);
    ws += kDecodeStatusBytes;
    a.arrivals = reinterpret_cast<uint32_t*>(ws);
    ws += align256((size_t)kDecodeMaxUnits * sizeof(uint32_t));
    a.part_o = reinterpret_cast<float*>(ws);
    ws += align256(slots * a.head_dim * sizeof(float));
    a.part_ml = reinterpret_cast<float*>(ws);
}

pakv_status pakv_decode_plan(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                             const int32_t* kv_lens, int32_t num_seqs, int32_t max_kv_len,
                             void* plan, size_t plan_bytes, void* stream) {
    clear_error();
    DecodeLaunch a;
    if (pakv_status s = decode_setup(map, layer, pages, num_seqs, max_kv_len, a)) return s;
    if (num_seqs == 0) return PAKV_OK;
    if (!kv_lens) return fail(PAKV_ERR_INVALID, "kv_lens is null");
    size_t need = decode_plan_bytes(map->layers[layer].desc, num_seqs, max_kv_len);
    if (!plan || plan_bytes < need)
        return fail(PAKV_ERR_WORKSPACE, "decode plan needs %zu bytes, got %zu", need, plan ? plan_bytes : (size_t)0);
    a.kv_lens = kv_lens;
    a.sched = static_cast<int32_t*>(plan);
    return hip_status(launch_decode_plan(a, stream), "decode_plan launch");
}

pakv_status pakv_paged_attn_decode_planned(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                           const void* plan, size_t plan_bytes, const void* q, void* out,
                                           int32_t num_seqs, int32_t max_kv_len,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    DecodeLaunch a;
    if (pakv_status s = decode_setup(map, layer, pages, num_seqs, max_kv_len, a)) return s;
    if (num_seqs == 0) return PAKV_OK;
    if (!q || !out) return fail(PAKV_ERR_INVALID, "q or out is null");
    const auto& d = map->layers[layer].desc;
    size_t need_plan = decode_plan_bytes(d, num_seqs, max_kv_len);
    if (!plan || plan_bytes < need_plan)
        return fail(PAKV_ERR_WORKSPACE, "decode plan needs %zu bytes, got %zu", need_plan,
                    plan ? plan_bytes : (size_t)0);
    size_t need = decode_partial_bytes(d, num_seqs);
    if (!workspace || workspace_bytes < need)
        return fail(PAKV_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.sched = const_cast<int32_t*>(static_cast<const int32_t*>(plan));
    bind_partials(a, workspace);
    return hip_status(launch_decode(a, stream), "paged_attn_decode launch");
}

pakv_status pakv_paged_attn_decode_append(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const void* plan, size_t plan_bytes, const void* k_new,
                                          const void* v_new, const void* q, void* out,
                                          int32_t num_seqs, int32_t max_kv_len,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    if (!layer_ok(map, layer)) return fail(PAKV_ERR_INVALID, "bad map or layer %d", layer);
    const auto& L = map->layers[layer];
    const bool owner = L.source == layer;
    if (owner && (L.desc.kv_dtype != PAKV_KV_BF16 || L.desc.k_eq_v))
        return fail(PAKV_ERR_UNSUPPORTED,
                    "append decode on an 8-bit or K=V layer is not built: store, then decode");
    if (owner && num_seqs > 0 && (!k_new || !v_new)) return fail(PAKV_ERR_INVALID, "k_new or v_new is null");
    DecodeLaunch a;
    if (pakv_status s = decode_setup(map, layer, pages, num_seqs, max_kv_len, a)) return s;
    if (num_seqs == 0) return PAKV_OK;
    if (!q || !out) return fail(PAKV_ERR_INVALID, "q or out is null");
    const auto& d = L.desc;
    size_t need_plan = decode_plan_bytes(d, num_seqs, max_kv_len);
    if (!plan || plan_bytes < need_plan)
        return fail(PAKV_ERR_WORKSPACE, "decode plan needs %zu bytes, got %zu", need_plan,
                    plan ? plan_bytes : (size_t)0);
    size_t need = decode_partial_bytes(d, num_seqs);
    if (!workspace || workspace_bytes < need)
        return fail(PAKV_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.sched = const_cast<int32_t*>(static_cast<const int32_t*>(plan));
    if (owner) {   // a shared layer's rows were stored by its source: a plain decode
        a.k_new = static_cast<const uint16_t*>(k_new);
        a.v_new = static_cast<const uint16_t*>(v_new);
        a.append = 1;
    }
    bind_partials(a, workspace);
    return hip_status(launch_decode(a, stream), "paged_attn_decode_append launch");
}

pakv_status pakv_paged_attn_decode(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                   const int32_t* kv_lens, const void* q, void* out,
                                   int32_t num_seqs, int32_t max_kv_len,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    DecodeLaunch a;
    if (pakv_status s = decode_setup(map, layer, pages, num_seqs, max_kv_len, a)) return s;
    if (num_seqs == 0) return PAKV_OK;
    if (!kv_lens || !q || !out) return fail(PAKV_ERR_INVALID, "kv_lens, q or out is null");
    const auto& d = map->layers[layer].desc;
    size_t need = decode_workspace_bytes(d, num_seqs, max_kv_len);
    if (!workspace || workspace_bytes < need)
        return fail(PAKV_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    a.kv_lens = kv_lens;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    bind_partials(a, workspace);
    a.sched = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + decode_partial_bytes(d, num_seqs));
    if (int e = launch_decode_plan(a, stream)) return hip_status(e, "decode_plan launch");
    return hip_status(launch_decode(a, stream), "paged_attn_decode launch");
}

pakv_status pakv_paged_attn_decode_noalloc(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                           const int32_t* kv_lens, const void* q, void* out,
                                           int32_t num_seqs, int32_t max_kv_len, void* stream) {
    clear_error();
    DecodeLaunch a;
    if (pakv_status s = decode_setup(map, layer, pages, num_seqs, max_kv_len, a)) return s;
    if (num_seqs == 0) return PAKV_OK;
    if (!kv_lens || !q || !out) return fail(PAKV_ERR_INVALID, "kv_lens, q or out is null");
    const auto& d = map->layers[layer].desc;
    const size_t need = decode_workspace_bytes(d, num_seqs, max_kv_len);
    if (need > kNoallocScratchBytes)
        return fail(PAKV_ERR_WORKSPACE,
                    "decode needs %zu bytes of workspace, above the %zu of the library's scratch: "
                    "call pakv_paged_attn_decode with a workspace", need, kNoallocScratchBytes);
    void* ws = nullptr;
    if (int e = noalloc_scratch(&ws)) return hip_status(e, "decode scratch address");
    a.kv_lens = kv_lens;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    bind_partials(a, ws);
    a.sched = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + decode_partial_bytes(d, num_seqs));
    a.zero_arrivals = 1;
    if (int e = launch_decode_plan(a, stream)) return hip_status(e, "decode_plan launch");
    return hip_status(launch_decode(a, stream), "paged_attn_decode_noalloc launch");
}

size_t pakv_decode_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

// Checks shared by the extend calls; k_ext / v_ext: the packed chunk rows (or
// null: the chunk is read from the slab).
// Whether a layer's extend needs staging for the bf16 kernel: 8-bit slabs,
// K=V layers and packed chunks do; a bf16 slab's own chunk does not.
static bool extend_needs_stage(const pakv_layer_map* map, int32_t layer, bool packed) {
    const auto& L = map->layers[layer];
    const auto& S = map->layers[L.source];
    return packed || L.desc.kv_dtype != PAKV_KV_BF16 || S.desc.k_eq_v;
}

// workspace (staged calls): null runs the layers that need staging on the
// general kernel; otherwise they are staged into it for the bf16 kernel
static pakv_status extend_call(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                               const int32_t* cu_q, const int32_t* prefix_lens, const void* q,
                               const void* k_ext, const void* v_ext, void* out,
                               int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_kv_len,
                               bool packed, void* stream, void* workspace = nullptr, size_t workspace_bytes = 0,
                               bool run_stage = true) {
    if (!layer_ok(map, layer)) return fail(PAKV_ERR_INVALID, "bad map or layer %d", layer);
    if (num_seqs < 0 || total_q < 0 || max_q_len < 0) return fail(PAKV_ERR_INVALID, "negative sizes");
    if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PAKV_OK;
    if (pakv_status s = check_pages(pages, num_seqs)) return s;
    if (max_kv_len < max_q_len) return fail(PAKV_ERR_INVALID, "max_kv_len below max_q_len");
    if ((int64_t)max_kv_len > (int64_t)pages->max_pages_per_seq * PAKV_PAGE_SIZE)
        return fail(PAKV_ERR_INVALID, "max_kv_len %d exceeds the page table's %d positions", max_kv_len,
                    pages->max_pages_per_seq * PAKV_PAGE_SIZE);
    if (!cu_q || !prefix_lens || !q || !out) return fail(PAKV_ERR_INVALID, "null pointer argument");
    const auto& L = map->layers[layer];
    const auto& S = map->layers[L.source];
    if (packed && (!k_ext || (!v_ext && !S.desc.k_eq_v)))
        return fail(PAKV_ERR_INVALID, "k_ext or v_ext is null");
    if (!S.bound) return fail(PAKV_ERR_INVALID, "slab of layer %d (source of %d) is not bound", L.source, layer);
    const int32_t group = L.desc.num_q_heads / L.desc.num_kv_heads;
    const bool stage = workspace != nullptr && extend_needs_stage(map, layer, packed);
    const bool fast = stage || (L.desc.kv_dtype == PAKV_KV_BF16 && !S.desc.k_eq_v && !packed);
    if (stage) {
        const size_t need = extend_stage_bytes(num_seqs, L.desc.num_kv_heads, L.desc.head_dim, L.desc.window,
                                               max_q_len, max_kv_len);
        if (workspace_bytes < need)
            return fail(PAKV_ERR_WORKSPACE, "workspace of %zu bytes, staging needs %zu", workspace_bytes, need);
    }
    // grid (Hkv, row blocks of 128 (fast) or 32 (general) (token, head) rows, sequences)
    const int64_t row_blocks = ((int64_t)max_q_len * group + (fast ? 127 : 31)) / (fast ? 128 : 32);
    if (row_blocks > 65535 || num_seqs > 65535)
        return fail(PAKV_ERR_UNSUPPORTED, "extend grid too large: %lld row blocks, %d sequences (65535 each at most)",
                    (long long)row_blocks, num_seqs);
    ExtendLaunch a;
    a.slab = view_of(S);
    a.page_table = pages->page_table;
    a.max_pages = pages->max_pages_per_seq;
    a.cu_q = cu_q;
    a.prefix_lens = prefix_lens;
    a.q = static_cast<const uint16_t*>(q);
    a.k_ext = packed ? static_cast<const uint16_t*>(k_ext) : nullptr;
    a.v_ext = packed && !S.desc.k_eq_v ? static_cast<const uint16_t*>(v_ext) : nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.max_kv_len = max_kv_len;
    a.hq = L.desc.num_q_heads;
    a.hkv = L.desc.num_kv_heads;
    a.head_dim = L.desc.head_dim;
    a.window = L.desc.window;
    a.sm_scale = L.desc.sm_scale;
    a.kv_dtype = L.desc.kv_dtype;
    a.k_eq_v = S.desc.k_eq_v;
    a.v_norm_eps = S.desc.v_norm_eps;
    if (stage) {
        if (run_stage)
            if (int e = launch_extend_stage(a, workspace, stream))
                return hip_status(e, "paged_attn_extend staging launch");
        // the bf16 kernel on the staged pages: the workspace is its slab
        const int32_t stride = extend_stage_stride(L.desc.window, max_q_len, max_kv_len);
        const int64_t blocks = (int64_t)num_seqs * stride * L.desc.num_kv_heads;
        auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
        char* w = static_cast<char*>(workspace);
        const int64_t page_bytes = al(blocks * 16 * L.desc.head_dim * 2);
        a.slab.k = w;
        a.slab.v = w + page_bytes;
        a.slab.k_scale = reinterpret_cast<const float*>(w + 2 * page_bytes);   // [Hkv][pages][32]
        a.slab.v_scale = nullptr;
        a.slab.num_pages = (int32_t)((int64_t)num_seqs * stride);
        a.stage_stride = stride;
        a.kv_dtype = PAKV_KV_BF16;
    }
    if (fast) return hip_status(launch_extend(a, stream), "paged_attn_extend launch");
    return hip_status(launch_extend_general(a, stream), "paged_attn_extend launch");
}

pakv_status pakv_paged_attn_extend(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                   const int32_t* cu_q, const int32_t* prefix_lens,
                                   const void* q, void* out,
                                   int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                   int32_t max_kv_len, void* stream) {
    clear_error();
    return extend_call(map, layer, pages, cu_q, prefix_lens, q, nullptr, nullptr, out, num_seqs, total_q, max_q_len,
                       max_kv_len, false, stream);
}

pakv_status pakv_paged_attn_extend_packed(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const int32_t* cu_q, const int32_t* prefix_lens,
                                          const void* q, const void* k_ext, const void* v_ext, void* out,
                                          int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, void* stream) {
    clear_error();
    return extend_call(map, layer, pages, cu_q, prefix_lens, q, k_ext, v_ext, out, num_seqs, total_q, max_q_len,
                       max_kv_len, true, stream);
}

size_t pakv_extend_staging_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_seqs, int32_t max_q_len,
                                  int32_t max_kv_len, int32_t packed) {
    if (!layer_ok(map, layer) || num_seqs <= 0 || max_q_len <= 0 || max_kv_len <= 0) return 0;
    if (!extend_needs_stage(map, layer, packed != 0)) return 0;
    const auto& d = map->layers[layer].desc;
    return extend_stage_bytes(num_seqs, d.num_kv_heads, d.head_dim, d.window, max_q_len, max_kv_len);
}

pakv_status pakv_paged_attn_extend_staged(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const int32_t* cu_q, const int32_t* prefix_lens,
                                          const void* q, const void* k_ext, const void* v_ext, void* out,
                                          int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                                          int32_t stage, void* stream) {
    clear_error();
    const bool packed = k_ext != nullptr;
    if (layer_ok(map, layer) && extend_needs_stage(map, layer, packed) && !workspace && num_seqs > 0 &&
        total_q > 0 && max_q_len > 0)
        return fail(PAKV_ERR_WORKSPACE, "null workspace: layer %d's extend is staged", layer);
    return extend_call(map, layer, pages, cu_q, prefix_lens, q, k_ext, v_ext, out, num_seqs, total_q, max_q_len,
                       max_kv_len, packed, stream, workspace, workspace_bytes, stage != 0);
}

pakv_status pakv_workgroup_xcds(int32_t* out, int32_t num_workgroups, void* stream) {
    clear_error();
    if (!out) return fail(PAKV_ERR_INVALID, "null pointer argument");
    if (num_workgroups < 1 || num_workgroups > 65535)
        return fail(PAKV_ERR_INVALID, "num_workgroups %d outside [1, 65535]", num_workgroups);
    return hip_status(launch_xcd_probe(out, num_workgroups, stream), "xcd probe launch");
}

}  // extern "C"

// The plans of two layers (of different kinds) from the same kv_lens, in one
// launch; the same checks as pakv_decode_plan for each.
pakv_status pakv::decode_plan_pair(const pakv_layer_map* map, const int32_t layer[2], const pakv_pages* const pages[2],
                                   const int32_t* kv_lens, int32_t num_seqs, int32_t max_kv_len,
                                   void* const plan[2], const size_t plan_bytes[2], void* stream) {
    clear_error();
    DecodeLaunch a[2];
    for (int k = 0; k < 2; ++k) {
        if (pakv_status s = decode_setup(map, layer[k], pages[k], num_seqs, max_kv_len, a[k])) return s;
        const size_t need = decode_plan_bytes(map->layers[layer[k]].desc, num_seqs, max_kv_len);
        if (!plan[k] || plan_bytes[k] < need)
            return fail(PAKV_ERR_WORKSPACE, "decode plan needs %zu bytes, got %zu", need,
                        plan[k] ? plan_bytes[k] : (size_t)0);
        a[k].kv_lens = kv_lens;
        a[k].sched = static_cast<int32_t*>(plan[k]);
    }
    if (num_seqs == 0) return PAKV_OK;
    if (!kv_lens) return fail(PAKV_ERR_INVALID, "kv_lens is null");
    return hip_status(launch_decode_plan2(a[0], a[1], stream), "decode_plan launch");
}

