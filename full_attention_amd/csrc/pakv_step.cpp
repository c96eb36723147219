// A decode step of a layer stack, captured into one HIP graph per batch-size
// bucket and replayed (unsloth commit dee9371: one CUDA graph per batch-size
// bucket; commit 749fb75: a single bucket ladder, a single pool across
// buckets).  The step is what a serving engine's decode runs for every layer:
// one plan per kind of layer (window, Hkv), then each layer's store of its new
// row and its decode, in layer order.  Every bucket's graph uses the same
// caller buffers (sized for the largest bucket) and the same workspace; a
// batch runs the graph of the smallest bucket that holds it, and the rows past
// the batch are decoded too, on whatever the caller keeps there.

#include <algorithm>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "pakv_internal.h"

struct pakv_decode_step {
    std::vector<int32_t> buckets;
    std::vector<hipGraphExec_t> execs;
};

namespace pakv {

// the step's kinds of layer: (window, Hkv) of the layers in first-seen order,
// with a representative layer each
struct StepKinds {
    std::vector<int32_t> rep;        // representative layer of kind k
    std::vector<int32_t> kind_of;    // kind of step layer i
};

static StepKinds step_kinds(const pakv_layer_map* map, const pakv_step_layer* layers, int32_t n) {
    StepKinds k;
    for (int32_t i = 0; i < n; ++i) {
        const auto& d = map->layers[layers[i].layer].desc;
        int32_t found = -1;
        for (size_t j = 0; j < k.rep.size(); ++j) {
            const auto& r = map->layers[k.rep[j]].desc;
            if (r.window == d.window && r.num_kv_heads == d.num_kv_heads) found = (int32_t)j;
        }
        if (found < 0) {
            found = (int32_t)k.rep.size();
            k.rep.push_back(layers[i].layer);
        }
        k.kind_of.push_back(found);
    }
    return k;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: [positions (cu 0..B, start kv_len - 1)] [plan of each kind] [decode workspace]
struct StepLayout {
    size_t pos, plans, ws, total;
    std::vector<size_t> plan_off, plan_bytes;
    size_t ws_bytes;
};

static StepLayout step_layout(const pakv_layer_map* map, const pakv_step_layer* layers, int32_t n, int32_t max_batch,
                              int32_t max_kv_len, const StepKinds& k) {
    StepLayout l;
    l.pos = 0;
    size_t off = align256((size_t)(2 * max_batch + 1) * sizeof(int32_t));
    l.plans = off;
    for (int32_t r : k.rep) {
        const size_t b = decode_plan_bytes(map->layers[r].desc, max_batch, max_kv_len);
        l.plan_off.push_back(off);
        l.plan_bytes.push_back(b);
        off += align256(b);
    }
    l.ws = off;
    l.ws_bytes = 0;
    for (int32_t i = 0; i < n; ++i)
        l.ws_bytes = std::max(l.ws_bytes, decode_partial_bytes(map->layers[layers[i].layer].desc, max_batch));
    l.total = off + align256(l.ws_bytes);
    return l;
}

}  // namespace pakv

using namespace pakv;

extern "C" {

size_t pakv_decode_step_workspace_bytes(const pakv_layer_map* map, const pakv_step_layer* layers, int32_t n_layers,
                                        int32_t max_batch, int32_t max_kv_len) {
    if (!map || !layers || n_layers <= 0 || max_batch <= 0 || max_kv_len < 1) return 0;
    for (int32_t i = 0; i < n_layers; ++i)
        if (layers[i].layer < 0 || layers[i].layer >= (int32_t)map->layers.size()) return 0;
    return step_layout(map, layers, n_layers, max_batch, max_kv_len, step_kinds(map, layers, n_layers)).total;
}

// Enqueues the step for a batch of B rows on stream s (captured by the caller).
static pakv_status enqueue_step(const pakv_layer_map* map, const pakv_pages* pages_full,
                                const pakv_pages* pages_sliding, const int32_t* kv_lens, int32_t B,
                                int32_t max_kv_len, const pakv_step_layer* layers, int32_t n,
                                const StepKinds& kinds, const StepLayout& lay, char* ws, void* s) {
    auto pages_of = [&](int32_t layer) {
        return map->layers[layer].desc.window > 0 && pages_sliding ? pages_sliding : pages_full;
    };
    int32_t* cu = reinterpret_cast<int32_t*>(ws + lay.pos);
    int32_t* start = cu + (B + 1);
    bool need_pos = false;
    for (int32_t i = 0; i < n; ++i) {
        const auto& L = map->layers[layers[i].layer];
        const bool owner = L.source == layers[i].layer;
        if (owner && layers[i].k_new && (L.desc.kv_dtype != PAKV_KV_BF16 || L.desc.k_eq_v)) need_pos = true;
    }
    if (need_pos)
        if (int e = launch_step_positions(kv_lens, B, cu, start, s)) return fail(PAKV_ERR_HIP, "step positions: %s",
                                                                                 hip_error_string(e));
    if (kinds.rep.size() == 2) {
        // both kinds' plans in one launch: they are independent, and each is
        // bound by its round trips rather than by its work
        const int32_t rep[2] = {kinds.rep[0], kinds.rep[1]};
        const pakv_pages* pg[2] = {pages_of(rep[0]), pages_of(rep[1])};
        void* const plans[2] = {ws + lay.plan_off[0], ws + lay.plan_off[1]};
        const size_t bytes[2] = {lay.plan_bytes[0], lay.plan_bytes[1]};
        if (pakv_status st = decode_plan_pair(map, rep, pg, kv_lens, B, max_kv_len, plans, bytes, s)) return st;
    } else {
        for (size_t k = 0; k < kinds.rep.size(); ++k) {
            const int32_t r = kinds.rep[k];
            if (pakv_status st = pakv_decode_plan(map, r, pages_of(r), kv_lens, B, max_kv_len, ws + lay.plan_off[k],
                                                  lay.plan_bytes[k], s))
                return st;
        }
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t l = layers[i].layer;
        const auto& L = map->layers[l];
        const bool owner = L.source == l;
        const int32_t k = kinds.kind_of[i];
        void* plan = ws + lay.plan_off[k];
        const size_t pb = lay.plan_bytes[k];
        pakv_status st;
        if (owner && layers[i].k_new && L.desc.kv_dtype == PAKV_KV_BF16 && !L.desc.k_eq_v) {
            st = pakv_paged_attn_decode_append(map, l, pages_of(l), plan, pb, layers[i].k_new, layers[i].v_new,
                                               layers[i].q, layers[i].out, B, max_kv_len, ws + lay.ws, lay.ws_bytes,
                                               s);
        } else {
            if (owner && layers[i].k_new) {
                st = pakv_paged_kv_store(map, l, pages_of(l), cu, start, layers[i].k_new, layers[i].v_new, B, B, s);
                if (st) return st;
            }
            st = pakv_paged_attn_decode_planned(map, l, pages_of(l), plan, pb, layers[i].q, layers[i].out, B,
                                                max_kv_len, ws + lay.ws, lay.ws_bytes, s);
        }
        if (st) return st;
    }
    return PAKV_OK;
}

void pakv_decode_step_destroy(pakv_decode_step* step) {
    if (!step) return;
    for (hipGraphExec_t e : step->execs)
        if (e) (void)hipGraphExecDestroy(e);
    delete step;
}

pakv_status pakv_decode_step_create(const pakv_layer_map* map, const pakv_pages* pages_full,
                                    const pakv_pages* pages_sliding, const int32_t* kv_lens, int32_t max_batch,
                                    int32_t max_kv_len, const pakv_step_layer* layers, int32_t n_layers,
                                    const int32_t* buckets, int32_t n_buckets, void* workspace,
                                    size_t workspace_bytes, pakv_decode_step** out) {
    clear_error();
    if (!out) return fail(PAKV_ERR_INVALID, "out is null");
    *out = nullptr;
    if (!map || !pages_full || !kv_lens || !layers || !buckets || !workspace)
        return fail(PAKV_ERR_INVALID, "null pointer argument");
    if (n_layers <= 0 || n_buckets <= 0 || max_batch <= 0 || max_kv_len < 1)
        return fail(PAKV_ERR_INVALID, "sizes must be positive");
    std::vector<int32_t> bk(buckets, buckets + n_buckets);
    std::sort(bk.begin(), bk.end());
    if (bk.front() < 1 || bk.back() > max_batch || std::unique(bk.begin(), bk.end()) != bk.end())
        return fail(PAKV_ERR_INVALID, "buckets must be distinct and within [1, max_batch]");
    for (int32_t i = 0; i < n_layers; ++i) {
        const int32_t l = layers[i].layer;
        if (l < 0 || l >= (int32_t)map->layers.size()) return fail(PAKV_ERR_INVALID, "step layer %d out of range", l);
        if (!layers[i].q || !layers[i].out) return fail(PAKV_ERR_INVALID, "step layer %d: q or out is null", l);
        const auto& L = map->layers[l];
        if (L.source == l && layers[i].k_new && !layers[i].v_new && !L.desc.k_eq_v)
            return fail(PAKV_ERR_INVALID, "step layer %d: k_new without v_new", l);
    }
    const StepKinds kinds = step_kinds(map, layers, n_layers);
    const StepLayout lay = step_layout(map, layers, n_layers, max_batch, max_kv_len, kinds);
    if (workspace_bytes < lay.total)
        return fail(PAKV_ERR_WORKSPACE, "decode step needs %zu bytes of workspace, got %zu", lay.total, workspace_bytes);
    pakv_decode_step* step = new (std::nothrow) pakv_decode_step;
    if (!step) return fail(PAKV_ERR_INVALID, "out of host memory");
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
        delete step;
        return fail(PAKV_ERR_HIP, "capture stream: %s", hipGetErrorString(hipGetLastError()));
    }
    pakv_status result = PAKV_OK;
    TimingPause pause;     // kernel timing events stay out of the graphs
    for (int32_t B : bk) {
        hipGraph_t g = nullptr;
        hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            result = fail(PAKV_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
            break;
        }
        pakv_status st = enqueue_step(map, pages_full, pages_sliding, kv_lens, B, max_kv_len, layers, n_layers, kinds,
                                      lay, static_cast<char*>(workspace), cs);
        e = hipStreamEndCapture(cs, &g);
        if (st || e != hipSuccess) {
            if (g) (void)hipGraphDestroy(g);
            result = st ? st : fail(PAKV_ERR_HIP, "end capture: %s", hipGetErrorString(e));
            break;
        }
        hipGraphExec_t ex = nullptr;
        e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) {
            result = fail(PAKV_ERR_HIP, "instantiate: %s", hipGetErrorString(e));
            break;
        }
        step->buckets.push_back(B);
        step->execs.push_back(ex);
    }
    (void)hipStreamDestroy(cs);
    if (result) {
        pakv_decode_step_destroy(step);
        return result;
    }
    *out = step;
    return PAKV_OK;
}

pakv_status pakv_decode_step_run(pakv_decode_step* step, int32_t batch, void* stream) {
    clear_error();
    if (!step) return fail(PAKV_ERR_INVALID, "step is null");
    if (batch <= 0) return PAKV_OK;
    for (size_t i = 0; i < step->buckets.size(); ++i) {
        if (step->buckets[i] >= batch) {
            const hipError_t e = hipGraphLaunch(step->execs[i], static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return fail(PAKV_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
            return PAKV_OK;
        }
    }
    return fail(PAKV_ERR_INVALID, "batch %d is larger than the largest bucket %d", batch, step->buckets.back());
}

int32_t pakv_decode_step_bucket(const pakv_decode_step* step, int32_t batch) {
    if (!step || batch <= 0) return -1;
    for (int32_t b : step->buckets)
        if (b >= batch) return b;
    return -1;
}

}  // extern "C"
