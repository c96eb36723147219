// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "pakv.h"

struct pakv_layer_map {
    struct Layer {
        pakv_layer_desc desc;
        int32_t source;     // layer whose slab this layer reads (itself for an owner)
        bool bound;         // a slab is attached (owners only)
        pakv_slab slab;
    };
    std::vector<Layer> layers;
};

namespace pakv {

pakv_status fail(pakv_status code, const char* fmt, ...);
void clear_error();

// ---- decode plan -------------------------------------------------------------
// Pass 1 runs a fixed grid of persistent workgroups (two per CU on a 256-CU
// part); the partition of the chunk stream depends only on the lengths.
constexpr int32_t kDecodeGrid = 512;
constexpr int32_t kDecodeMaxSeqs = 1023;     // sequences per decode call
constexpr int32_t kDecodeMaxUnits = 8192;    // num_seqs * Hkv per decode call
constexpr size_t kDecodeStatusBytes = 256;   // the workspace's first block: the status word
struct DecodePlan {
    int32_t grid;           // workgroups of pass 1
    int32_t units;          // num_seqs * Hkv
    int32_t group;          // Hq / Hkv
};
DecodePlan plan_decode(const pakv_layer_desc& d, int32_t num_seqs);

// The schedule of a decode call (pakv_decode_plan), a device buffer of int32
// words written by the plan kernel from kv_lens and the page table and read by
// the decode kernel, so that a decode workgroup learns its run of the chunk
// stream and the first page ids in one load:
//   [0, kPlanHeader)   magic, total chunks T, chunks per workgroup (0 for
//                      the unit-aligned split), grid, B, Hkv, window, max_kv_len
//   soff [B + 1]       first stream chunk of each sequence's units; soff[B] = T
//   slen [B]           length of each sequence, clamped to [1, max_kv_len]
//   rec  [grid][kPlanRecord]  per decode workgroup i, the record of the run
//                      w it takes (when grid is a multiple of 8, XCD i mod 8
//                      takes a block of consecutive runs: grid / 8 of them for
//                      stream-K, an even share of the busy runs for the
//                      aligned split): first chunk, end chunk, unit of the
//                      first chunk, that chunk's index in its unit, chunks per
//                      run (0 for the unit-aligned split), the first and last
//                      run of its unit (aligned split only), w, whether the
//                      unit's runs lie in one XCD's block (aligned split
//                      only), spare words, then from word kPlanRecIds the page
//                      ids of its first 64 chunks (-1 past its run)
//   ids  [cap]         page id of every stream chunk (ids outside the pool
//                      replaced by -1: read as page 0, never written)
constexpr int32_t kPlanMagic = 0x31504b50;
constexpr int32_t kPlanHeader = 16;
constexpr int32_t kPlanRecord = 80;
constexpr int32_t kPlanRecIds = 16;
struct PlanLayout {
    int64_t soff, slen, rec, ids;   // word offsets
    int64_t cap;                    // chunk capacity of ids
    int64_t words;
};
PlanLayout plan_layout(int32_t num_seqs, int32_t hkv, int32_t max_kv_len);
size_t decode_plan_bytes(const pakv_layer_desc& d, int32_t num_seqs, int32_t max_kv_len);
// partials and arrival counters; the unplanned call also keeps its plan there
size_t decode_partial_bytes(const pakv_layer_desc& d, int32_t num_seqs);
size_t decode_workspace_bytes(const pakv_layer_desc& d, int32_t num_seqs, int32_t max_kv_len);

// ---- launchers (defined in the .hip translation units) ----------------------
struct SlabView {
    const void* k;
    const void* v;
    const float* k_scale;
    const float* v_scale;
    int32_t num_pages;
};

struct StoreLaunch {
    SlabView slab;          // written through the const-casted pointers
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_tokens;
    const int32_t* start_pos;
    const uint16_t* k;
    const uint16_t* v;      // null for a K=V layer
    int32_t num_seqs;
    int32_t total_tokens;
    int32_t hkv;
    int32_t head_dim;
    int32_t kv_dtype;
};
int launch_store(const StoreLaunch& a, void* stream);   // returns hipError_t

struct DecodeLaunch {
    SlabView slab;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* kv_lens;
    const uint16_t* q;
    uint16_t* out;
    int32_t num_seqs;
    int32_t max_kv_len;
    int32_t hq;
    int32_t hkv;
    int32_t head_dim;
    int32_t window;
    int32_t kv_dtype;
    int32_t k_eq_v;         // values are the RMS-normalised keys (K slab only)
    float v_norm_eps;
    float sm_scale;
    DecodePlan plan;
    int32_t* sched;     // the schedule buffer (written by the plan kernel, read by the decode kernel)
    PlanLayout layout;
    uint32_t* status;   // sticky status word (workspace offset 0)
    uint32_t* arrivals; // [units], zero between calls
    float* part_o;      // [grid + units][G][D]
    float* part_ml;     // [grid + units][G][2]
    const uint16_t* k_new = nullptr;   // append: [num_seqs][hkv][D] bf16, stored at kv_len - 1
    const uint16_t* v_new = nullptr;
    int32_t append = 0;
    int32_t zero_arrivals = 0;   // the plan kernel zeroes the call's counters first
    int32_t check_xcd = 0;       // pakv_set_decode_checks(PAKV_CHECK_XCD_PLACEMENT)
};
int launch_decode_plan(const DecodeLaunch& a, void* stream);   // writes a.sched from kv_lens, page_table
// two plans (a decode step's two kinds of layer, same kv_lens) in one launch
int launch_decode_plan2(const DecodeLaunch& a0, const DecodeLaunch& a1, void* stream);
pakv_status decode_plan_pair(const pakv_layer_map* map, const int32_t layer[2], const pakv_pages* const pages[2],
                             const int32_t* kv_lens, int32_t num_seqs, int32_t max_kv_len, void* const plan[2],
                             const size_t plan_bytes[2], void* stream);
int launch_decode(const DecodeLaunch& a, void* stream);        // reads a.sched
int launch_xcd_probe(int32_t* out, int32_t n, void* stream);  // out[i] = XCD of workgroup i

// The library's own decode workspace, for pakv_paged_attn_decode_noalloc: a
// static device array of kNoallocScratchBytes on every GPU the library runs
// on.  noalloc_scratch() returns the current device's address of it (taken
// once per device with hipGetSymbolAddress); a hipError_t, 0 on success.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
constexpr int kNoallocMaxDevices = 64;
int noalloc_scratch(void** ptr);

// The counters of a PAKV_DEBUG_BOUNDS build (uint32_t[kDebugCounters], a
// file-scope device array): the current device's address, taken once per
// device; null in other builds, and on error.
constexpr int kDebugCounters = 4;
uint32_t* debug_bad_ids_ptr();
int debug_bad_ids_read(uint32_t* out, int n);   // waits for the device; hipError_t
int debug_bad_ids_reset();                      // waits for the device; hipError_t

struct ExtendLaunch {
    SlabView slab;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_q;
    const int32_t* prefix_lens;
    const uint16_t* q;
    const uint16_t* k_ext = nullptr;   // packed chunk rows [total_q][Hkv][D], or null (chunk read from the slab)
    const uint16_t* v_ext = nullptr;
    uint16_t* out;
    int32_t num_seqs;
    int32_t total_q;
    int32_t max_q_len;
    int32_t max_kv_len;
    int32_t hq;
    int32_t hkv;
    int32_t head_dim;
    int32_t window;
    float sm_scale;
    int32_t kv_dtype = PAKV_KV_BF16;
    int32_t k_eq_v = 0;
    float v_norm_eps = 0.f;
    // the bf16 kernel on staged pages (slab = the staging workspace, with
    // k_scale / v_scale its per-token scales), pages per sequence; 0 otherwise
    int32_t stage_stride = 0;
};
int launch_extend(const ExtendLaunch& a, void* stream);           // bf16 K and V slabs (or staged pages)
int launch_extend_general(const ExtendLaunch& a, void* stream);   // 8-bit, K=V, packed chunks
// staging of a call's visible keys and values for the bf16 kernel
// (kernels_extend_stage.hip): pages per sequence, workspace bytes, the pass
int32_t extend_stage_stride(int32_t window, int32_t max_q_len, int32_t max_kv_len);
size_t extend_stage_bytes(int32_t num_seqs, int32_t hkv, int32_t head_dim, int32_t window, int32_t max_q_len,
                          int32_t max_kv_len);
int launch_extend_stage(const ExtendLaunch& a, void* workspace, void* stream);

const char* hip_error_string(int err);

// pakv_set_decode_checks flags, read when a decode call is set up
int32_t decode_checks();

// Timing hook (pakv_set_timing_events): the next event-pair index for a kernel
// selected by `kind` (a PAKV_TIME_* bit), or -1; and the caller's event array.
int timing_slot(int kind);
void* const* timing_events();
// Switches the hook off on this thread for the object's lifetime (graph
// capture: event records inside a graph do not bracket its kernels).
struct TimingPause {
    TimingPause();
    ~TimingPause();
    void* const* events;
    int32_t pairs, used, mask;
};

// cu[b] = b (b <= B) and start[b] = kv_lens[b] - 1 (b < B): the store
// arguments of one new row per sequence, for a decode step.
int launch_step_positions(const int32_t* kv_lens, int32_t B, int32_t* cu, int32_t* start, void* stream);

}  // namespace pakv
