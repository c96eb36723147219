// paged_attn_decode: split-KV decode with a deterministic combine.
//
// Pass 1 (partial): the work of all (sequence b, KV head g) units is a
// stream of 16-token chunks (one page each): unit (b, g) covers the pages
// that hold its visible keys [lo, L).  A fixed grid of persistent workgroups
// (4 wavefronts each) takes contiguous runs of that stream of at most a
// common length: split unit by unit when every unit can have workgroups of
// its own (no run then crosses a unit), else equal pieces of the stream
// (stream-K), so every workgroup moves about the same bytes whatever the
// length mix.  A run that crosses unit boundaries produces one partial
// (o, m, l) per unit it touches, stored at slot (workgroup + unit).  Chunks are streamed into
// LDS by asynchronous global->LDS copies (global_load_lds_dwordx4), NBUF deep,
// so the bytes in flight hold no registers.  For each chunk:
//
//   S^T[16 tokens x 16 heads] = K_page . Q_g^T   each wavefront contracts its
//                               own quarter of D (MFMA 16x16x32); the four
//                               partial scores are summed through LDS in a
//                               fixed order, so every wavefront holds the same
//                               scores
//   online softmax per head column (exp2 domain)
//   O^T[D/4 x 16 heads]      += V_page^T . P^T  each wavefront owns a quarter
//                               of the output dims (MFMA 16x16x16)
//
// The G query heads that share KV head g are the 16 MFMA columns (columns >= G
// are zero padding), so every K/V byte is read from HBM once per (sequence, KV
// head).  V pages are dim-major, so the value product's operand (one dim, four
// consecutive tokens) is one 8-byte LDS read.
//
// Combine: the workgroup that finishes a unit's last partial (a per-unit
// arrival counter; the merging workgroup resets it to zero) merges the unit's
// partials.  The dispatcher places workgroup i on XCD i mod 8 (the same class
// of i mod 8 shares an XCD also when a partition has 1, 2 or 4 XCDs), and the
// plan's workgroup numbering gives each XCD a contiguous block of runs; a
// unit whose runs all fall in one block exchanges its partials through that
// XCD's L2, the others through memory.  The merge goes in workgroup order: M = max_s m_s,
// O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, rounded to bf16.  Which
// workgroup merges does not change the arithmetic, no atomics touch
// floating-point data, and the partition depends only on the lengths, so
// results are bit-identical run to run and do not depend on page placement.
//
// Masks (unsloth commit ca9dbce, one block mask per regime): the decode query
// sits at position L - 1 (L = kv_lens[b]); keys [lo, L) are visible with
// lo = 0 for a full layer and lo = max(0, L - W) for a sliding one.  Scores of
// other keys are selected to -inf, and their value elements are selected to
// zero before the product (slots that were never written may hold NaN).

#include <mutex>

#include "async_copy.h"
#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 16;        // tokens per staged chunk (one page)
constexpr uint32_t kNoPage = 0xffffffffu;   // a chunk whose page id lies outside the pool
// status word bits (sticky: set by a call that detects the condition, cleared
// only by the caller)
constexpr uint32_t kStatusPlanMismatch = 1u;    // the plan was made for another shape
constexpr uint32_t kStatusXcdSplit = 2u;        // an XCD-local unit's workgroups ran on several XCDs

struct DecodeArgs {
    const uint8_t* k_slab;
    const uint8_t* v_slab;
    const float* k_scale;
    const float* v_scale;
    int32_t num_pages;
    int32_t max_pages;
    const uint16_t* q;
    uint16_t* out;
    int32_t num_seqs;
    int32_t hq;
    int32_t hkv;
    int32_t group;
    int32_t window;
    float score_scale;      // sm_scale * log2(e)
    int32_t max_kv_len;
    int32_t grid;           // workgroups
    int32_t* sched;         // schedule buffer (word offsets below)
    int64_t s_soff, s_slen, s_rec, s_ids, s_cap;
    uint32_t* status;       // sticky status word (kStatus* bits), read by the caller
    uint32_t* arrivals;     // [U] partials written per unit; zero between calls
    float* part_o;          // [grid + U][G][D]
    float* part_ml;         // [grid + U][G][2]
    // append (bf16 slabs only): this step's K/V row of each (sequence, KV
    // head), [B][Hkv][D], stored at position L - 1 and attended as that key
    const uint16_t* k_new;
    const uint16_t* v_new;
    int32_t append;
    // set by the call that uses the library's own scratch: the plan kernel
    // zeroes the arrival counters of the call's units first
    int32_t zero_arrivals;
    float v_norm_eps;       // K=V layers: eps under the root of the value norm
    int32_t check_xcd;      // flag and check the XCDs of units merged inside one XCD
    uint32_t* bad_ids;      // counters of a PAKV_DEBUG_BOUNDS build, else null
};

// Waits for this wave's copies so that at most `newer` chunks' copies stay in
// flight (newer <= NBUF - 2).
template <int PER, int NBUF>
__device__ __forceinline__ void wait_chunks(int newer) {
    if constexpr (NBUF >= 5) { if (newer >= 3) { wait_vm<3 * PER>(); return; } }
    if constexpr (NBUF >= 4) { if (newer >= 2) { wait_vm<2 * PER>(); return; } }
    if constexpr (NBUF >= 3) { if (newer >= 1) { wait_vm<PER>(); return; } }
    wait_vm<0>();
}

// KV formats of the decode kernel (template argument F): bf16 K and V slabs;
// int8 or fp8 (E4M3) codes with a float32 scale per token and head; bf16 K
// only, the values being the RMS-normalised keys (K=V layers).
constexpr int kFmtBF16 = 0, kFmtINT8 = 1, kFmtFP8 = 2, kFmtKEQV = 3;

template <int D, int F>
struct Cfg {
    static constexpr bool Q8 = F == kFmtINT8 || F == kFmtFP8;   // 8-bit codes with scales
    static constexpr bool HAS_V = F != kFmtKEQV;             // a V slab to copy
    static constexpr int ES = Q8 ? 1 : 2;                   // bytes per code
    static constexpr int ROW = D * ES;                      // bytes per K row
    static constexpr int PAGE = 16 * D * ES;                // bytes per (page, head) block
    static constexpr int SCALE_BYTES = Q8 ? 128 : 0;        // k and v scales of one page
    static constexpr int BUF = (HAS_V ? 2 : 1) * PAGE + SCALE_BYTES;
    // ring slots: bf16 pages copied one ahead (two slots); a deeper ring
    // (three or four slots at D = 256) was slower in the step: with every
    // workgroup streaming, more requests in flight only lengthen the queues
    // and the stragglers.  int8 pages are half the bytes: four slots.
    static constexpr int NBUF = Q8 ? 4 : 2;
    static constexpr int KV_DMA = (HAS_V ? 2 : 1) * PAGE / (1024 * kWaves);   // copies per wave per chunk
    static constexpr int PER = KV_DMA + (Q8 ? 1 : 0);
    // partial-score exchange (and, for K=V, each wave's partial sums of
    // squares of the 16 key rows)
    static constexpr int SX = kWaves * 64 * 16 + (HAS_V ? 0 : kWaves * 16 * 4);
    static constexpr int SEQ = (2 * (pakv::kDecodeMaxSeqs + 1) * 4 + 15) & ~15;   // per-sequence table
    // append: per ring slot, the new V row (D bf16) and the page id it goes to
    static constexpr int STAGE = F == kFmtBF16 ? D * 2 : 0;
    static constexpr int NEWP = F == kFmtBF16 ? 16 : 0;
    static constexpr int LDS = NBUF * BUF + SX + SEQ + NBUF * STAGE + NEWP;
    static constexpr int KK = D / 128;                      // 32-dim steps in a wave's quarter
    static constexpr int MT = D / 64;                       // 16-dim output tiles in a quarter
    static_assert(LDS <= 80 * 1024, "two workgroups per CU");
};

// Per-sequence table in LDS, built once per workgroup from kv_lens:
//   soff[b] = first chunk of sequence b's units (units of a sequence are
//             consecutive, one per KV head, each n_b chunks), soff[B] = total
//   slen[b] = clamped length of sequence b
struct SeqTable {
    int32_t* soff;   // [B + 1]
    int32_t* slen;   // [B]
};

// Chunks of a unit: pages from lo/16 to (L-1)/16.
struct Unit {
    int32_t u, b, g, lo, hi, page0, n, first;   // first = stream index of its chunk 0
};

__device__ __forceinline__ int32_t window_lo(const DecodeArgs& a, int32_t len) {
    return (a.window > 0 && len > a.window) ? len - a.window : 0;
}

__device__ __forceinline__ int32_t chunks_of(const DecodeArgs& a, int32_t len) {
    return ((len + 15) >> 4) - (window_lo(a, len) >> 4);
}

__device__ __forceinline__ Unit unit_of(const DecodeArgs& a, const SeqTable& st, int32_t u) {
    Unit x;
    x.u = u;
    x.b = u / a.hkv;
    x.g = u - x.b * a.hkv;
    x.hi = st.slen[x.b];
    x.lo = window_lo(a, x.hi);
    x.page0 = x.lo >> 4;
    x.n = ((x.hi + 15) >> 4) - x.page0;
    x.first = st.soff[x.b] + x.g * x.n;
    return x;
}

// Sequence holding stream chunk c: the last b with soff[b] <= c.
__device__ __forceinline__ int32_t seq_of_chunk(const SeqTable& st, int32_t B, int32_t c) {
    int32_t lo = 0, hi = B - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (st.soff[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ void advance(const DecodeArgs& a, const SeqTable& st, int32_t U, Unit& x, int32_t& k) {
    if (++k == x.n && x.u + 1 < U) {
        x = unit_of(a, st, x.u + 1);
        k = 0;
    }
}

__device__ __forceinline__ void build_seq_table(const DecodeArgs& a, const int32_t* __restrict__ kv_lens,
                                                const SeqTable& st, int32_t B) {
    __shared__ int32_t wave_tot[kWaves];
    const int t = threadIdx.x;
    const int per_t = (B + 255) / 256;
    const int b0 = t * per_t, b1 = min(b0 + per_t, B);
    int32_t local = 0;
    for (int b = b0; b < b1; ++b) {
        const int32_t len = clamp_i32(kv_lens[b], 1, a.max_kv_len);
        st.slen[b] = len;
        local += chunks_of(a, len) * a.hkv;
    }
    int32_t incl = local;
    const int lane = t & 63, wave = t >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    int32_t run = before + incl - local;
    for (int b = b0; b < b1; ++b) {
        st.soff[b] = run;
        run += chunks_of(a, st.slen[b]) * a.hkv;
    }
    if (t == 255) st.soff[B] = before + incl;
    __syncthreads();
}

// Page id of stream chunk c: the page of sequence b holding the chunk's 16
// keys.  Ids outside the pool become kNoPage: the decode kernel reads page 0
// in their place (so a bad table never makes a copy leave the slab) and an
// append never writes to them.
__device__ __forceinline__ uint32_t page_of_chunk(const DecodeArgs& a, const int32_t* __restrict__ page_table,
                                                  const SeqTable& st, int32_t B, int32_t c) {
    const int32_t b = seq_of_chunk(st, B, c);
    const int32_t len = st.slen[b];
    const int32_t n = chunks_of(a, len);
    const int32_t k = (c - st.soff[b]) % n;
    const int32_t ph = page_table[(int64_t)b * a.max_pages + (window_lo(a, len) >> 4) + k];
    if ((uint32_t)ph < (uint32_t)a.num_pages) return (uint32_t)ph;
    note_bad_id(a.bad_ids, kBadIdPlan);
    return kNoPage;
}

// Prefix over sequences of the decode workgroups an aligned split gives them
// (ws[b]; ws[B] = total): every unit of sequence b, n_b chunks, gets
// ceil(n_b / per) workgroups, so that no run crosses a unit.
__device__ __forceinline__ void build_wg_table(const DecodeArgs& a, const SeqTable& st, int32_t B, int32_t per,
                                               int32_t* ws) {
    __shared__ int32_t wave_tot[kWaves];
    const int t = threadIdx.x;
    const int per_t = (B + 255) / 256;
    const int b0 = t * per_t, b1 = min(b0 + per_t, B);
    int32_t local = 0;
    for (int b = b0; b < b1; ++b) local += a.hkv * ((chunks_of(a, st.slen[b]) + per - 1) / per);
    int32_t incl = local;
    const int lane = t & 63, wave = t >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    int32_t run = before + incl - local;
    for (int b = b0; b < b1; ++b) {
        ws[b] = run;
        run += a.hkv * ((chunks_of(a, st.slen[b]) + per - 1) / per);
    }
    if (t == 255) ws[B] = before + incl;
    __syncthreads();
}

// The schedule of a decode call (the plan): every workgroup of a plan builds
// the sequence table, takes run w (its index among the plan's grid
// workgroups) of the chunk stream and writes its record (at the decode
// workgroup that will stream it) and the page ids of its chunks; the
// workgroup of run 0 also writes the header and the table.
//
// Runs hold at most per chunks.  When giving every unit its own
// ceil(n / per) workgroups fits the grid for some per no more than a half
// above ceil(T / grid) (units few, or of similar length, like a sliding
// window's), each unit is split evenly over its own workgroups and no run
// crosses a unit: a run that crosses one writes two partials and reloads Q in
// mid-stream, and those workgroups were the last to finish.  Otherwise runs
// are equal contiguous pieces of ceil(T / grid) chunks (stream-K).  Record fields: c_begin, c_end, first unit, its first
// chunk, then per for stream-K, or 0 and the first and last workgroup of the
// unit for the aligned split.
__device__ __forceinline__ void plan_body(const DecodeArgs& a, const int32_t* __restrict__ page_table,
                                          const int32_t* __restrict__ kv_lens, int32_t w, int32_t n_wg) {
    __shared__ int32_t seq_lds[2 * (pakv::kDecodeMaxSeqs + 1)];
    __shared__ int32_t ws_lds[pakv::kDecodeMaxSeqs + 1];
    const SeqTable st{seq_lds, seq_lds + pakv::kDecodeMaxSeqs + 1};
    const int t = threadIdx.x;
    const int32_t B = a.num_seqs;
    if (a.zero_arrivals) {
        // the decode kernel runs after this kernel ends (stream order), and
        // counts its arrivals from zero
        for (int32_t i = w * 256 + t; i < B * a.hkv; i += n_wg * 256) a.arrivals[i] = 0u;
    }
    build_seq_table(a, kv_lens, st, B);
    const int32_t T = st.soff[B];
    // the aligned split may lengthen the longest run by up to a half (at
    // least one chunk): the full layers of the E2B-like step need one more
    // chunk per run to align, and gain (59.7 -> 58.0 us); the 26B-like
    // sliding layers (units of 65 chunks, 49 per run even) take one run per
    // unit at 65 and merge nothing, instead of stream-K runs that each cross
    // a unit (step 2.66 -> 2.56 ms)
    const int32_t per0 = max((T + a.grid - 1) / a.grid, 1);
    int32_t per = per0;
    bool aligned = false;
    // Small batches (under 4 chunks per workgroup on average): filling the
    // grid cut a unit into as many runs as it has chunks, and its merging
    // workgroup then read them all, 7 or 8 per round trip.  The runs of a
    // unit are capped (16 on sliding layers, whose units are short, 32 on
    // full ones), measured over the batch buckets of the E2B-like step:
    // batch 1 0.565 -> 0.380 ms, batch 8 0.587 -> 0.417 ms, batch 16
    // 0.566 -> 0.500 ms per step; 32 and 64 unchanged.
    int32_t p_min = per0;
    if (per0 < 4) {
        __shared__ int32_t nmax_w[kWaves];
        int32_t m = 0;
        for (int32_t b = t; b < B; b += 256) m = max(m, chunks_of(a, st.slen[b]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
        if ((t & 63) == 0) nmax_w[t >> 6] = m;
        __syncthreads();
        int32_t nmax = nmax_w[0];
        for (int w2 = 1; w2 < kWaves; ++w2) nmax = max(nmax, nmax_w[w2]);
        const int32_t cap = a.window > 0 ? 16 : 32;
        p_min = max(per0, (nmax + cap - 1) / cap);
    }
    for (int32_t p = p_min; p <= p_min + max(p_min / 2, 1); ++p) {
        build_wg_table(a, st, B, p, ws_lds);
        if (ws_lds[B] <= a.grid) {
            aligned = true;
            per = p;
            break;
        }
    }
    int32_t c_begin, c_end, u = 0, kc = 0, rw0 = 0, rw1 = 0;
    if (aligned) {
        c_begin = c_end = T;
        if (w < ws_lds[B]) {
            int32_t lo = 0, hi = B - 1;                 // sequence b: the last with ws[b] <= w
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (ws_lds[mid] <= w) lo = mid; else hi = mid - 1;
            }
            const int32_t b = lo;
            const int32_t n = chunks_of(a, st.slen[b]);
            const int32_t nw = (n + per - 1) / per;     // workgroups per unit of b
            const int32_t r = w - ws_lds[b], g = r / nw, k = r % nw;
            const int32_t first = st.soff[b] + g * n;
            u = b * a.hkv + g;
            kc = (k * n) / nw;
            c_begin = first + kc;
            c_end = first + ((k + 1) * n) / nw;
            rw0 = ws_lds[b] + g * nw;
            rw1 = rw0 + nw - 1;
        }
    } else {
        per = per0;
        c_begin = min(w * per, T);
        c_end = min(c_begin + per, T);
        if (c_begin < c_end) {
            const int32_t b = seq_of_chunk(st, B, c_begin);
            const int32_t n = chunks_of(a, st.slen[b]);
            const int32_t r = c_begin - st.soff[b];
            u = b * a.hkv + r / n;
            kc = r % n;
        }
    }
    int32_t* S = a.sched;
    if (w == 0) {
        if (t == 0) {
            const int32_t head[8] = {pakv::kPlanMagic, T, aligned ? 0 : per, a.grid, B, a.hkv, a.window,
                                     a.max_kv_len};
#pragma unroll
            for (int i = 0; i < 8; ++i) S[i] = head[i];
        }
        for (int i = t; i <= B; i += 256) S[a.s_soff + i] = st.soff[i];
        for (int i = t; i < B; i += 256) S[a.s_slen + i] = st.slen[i];
    }
    // The record goes to the decode workgroup that runs this run.  The
    // dispatcher puts decode workgroup i on XCD i mod 8, so XCD x runs the
    // workgroups x, x + 8, ...; each XCD is given a block of consecutive runs.
    // Stream-K: blocks of grid / 8 runs.  Aligned split: the R runs are shared
    // out evenly, block x = [R x / 8, R (x + 1) / 8): with blocks of grid / 8
    // a sliding layer's 448 runs left one XCD idle (E2B-like step 0.759 ->
    // 0.755 ms; boundaries moved to unit boundaries, which keeps every merge
    // inside one XCD but unbalances the blocks, measured slower).
    // The idle workgroups of each XCD take the runs past R (empty records).
    // An aligned record also says whether its unit's runs lie in one block
    // (then the unit's partials stay in that XCD's L2).
    const int32_t xblk = (a.grid & 7) == 0 ? a.grid >> 3 : 0;
    int32_t dst = w, local = 0;
    if (xblk > 0 && !aligned) {
        dst = (w % xblk) * 8 + w / xblk;
    } else if (xblk > 0) {
        const int32_t R = ws_lds[B];                  // <= grid, so R * 8 cannot overflow
        auto block_start = [&](int32_t x) { return (R * x) >> 3; };
        auto block_of = [&](int32_t r) {
            int32_t x = 7;
            while (x > 0 && block_start(x) > r) --x;
            return x;
        };
        if (w < R) {
            const int32_t x = block_of(w);
            dst = (w - block_start(x)) * 8 + x;
            local = block_of(rw0) == block_of(rw1) ? 1 : 0;
        } else {
            int32_t k = w - R;
            for (int32_t x = 0; x < 8; ++x) {
                const int32_t n = block_start(x + 1) - block_start(x);
                if (k < xblk - n) {
                    dst = (n + k) * 8 + x;
                    break;
                }
                k -= xblk - n;
            }
        }
    }
    int32_t* rec = S + a.s_rec + (int64_t)dst * pakv::kPlanRecord;
    if (t == 0) {
        rec[0] = c_begin;
        rec[1] = c_end;
        rec[2] = u;
        rec[3] = kc;
        rec[4] = aligned ? 0 : per;
        rec[5] = rw0;
        rec[6] = rw1;
        rec[7] = w;
        rec[8] = local;
    }
    for (int32_t j = t; j < max(c_end - c_begin, 64); j += 256) {
        const bool in_run = c_begin + j < c_end;
        const uint32_t id = in_run ? page_of_chunk(a, page_table, st, B, c_begin + j) : kNoPage;
        if (j < 64) rec[pakv::kPlanRecIds + j] = (int32_t)id;
        if (in_run) S[a.s_ids + c_begin + j] = (int32_t)id;
    }
}

// One plan (workgroup w takes run w), or the two plans of a decode step's two
// kinds of layer in one launch (the first grid's workgroups take the first;
// the plans are independent and each alone is bound by its round trips).
// Each calls the body with its own kernel parameters.
__global__ __launch_bounds__(256) void decode_plan_kernel(DecodeArgs a, const int32_t* __restrict__ page_table,
                                                           const int32_t* __restrict__ kv_lens) {
    plan_body(a, page_table, kv_lens, (int32_t)blockIdx.x, (int32_t)gridDim.x);
}

__global__ __launch_bounds__(256) void decode_plan2_kernel(DecodeArgs a0, DecodeArgs a1,
                                                            const int32_t* __restrict__ page_table0,
                                                            const int32_t* __restrict__ page_table1,
                                                            const int32_t* __restrict__ kv_lens) {
    if ((int32_t)blockIdx.x < a0.grid) plan_body(a0, page_table0, kv_lens, (int32_t)blockIdx.x, a0.grid);
    else plan_body(a1, page_table1, kv_lens, (int32_t)blockIdx.x - a0.grid, a1.grid);
}

// Page ids of stream chunks c0 .. c0 + count - 1 from the schedule (lane j
// holds chunk c0 + j; lanes past `count` hold kNoPage), as the plan wrote
// them: the copies clamp them to the pool (issue_chunk).
// (The lane index is made opaque here so that the address is formed where it
// is used, once per 64 chunks, instead of being held in registers all along.)
__device__ __forceinline__ uint32_t sched_ids(const DecodeArgs& a, int32_t c0, int32_t count, int lane) {
    asm volatile("" : "+v"(lane));
    uint32_t id = kNoPage;
    if (lane < count && c0 + lane < a.s_cap) id = (uint32_t)a.sched[a.s_ids + c0 + lane];
    return id;
}

// Q^T operand of a wave's dim quarter: column `col` = head g*G + col (zero
// for padding columns), dims dq + 32*kk + 8*qg .. +8.  The loads are inline
// assembly, so the compiler does not track them: a tracked load of Q that is
// still pending where the loop begins makes it wait on the vector-memory
// counter before every use of Q inside the loop, which (that counter being
// in order) drains every copy in flight on every chunk.  They are issued
// before a chunk's copies and complete before them; take_q() then hands the
// registers to the compiler, after the wait that covers them.
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, const Unit& x, int32_t G, int col, int qg, int dq,
                                       u32x4 (&qreg)[D / 128]) {
    const uint16_t* qp = a.q + ((int64_t)x.b * a.hq + (int64_t)x.g * G + (col < G ? col : 0)) * D + dq + 8 * qg;
#pragma unroll
    for (int kk = 0; kk < D / 128; ++kk)
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(qreg[kk]) : "v"(qp + 32 * kk) : "memory");
}

template <int N>
__device__ __forceinline__ void take_q(u32x4 (&qreg)[N], bool real) {
#pragma unroll
    for (int kk = 0; kk < N; ++kk) {
        asm volatile("" : "+v"(qreg[kk]));
        if (!real) qreg[kk] = u32x4{0, 0, 0, 0};
    }
}

// Copies of a chunk into a ring slot.  In an append call, a unit's last
// chunk holds the new key at position L - 1, whose row in the slab is not
// written yet: the page's copy skips K row r = (L - 1) % 16, which the wave
// that owns it copies from k_new instead (same swizzle, so no two copies
// write the same LDS bytes), and wave 0 first stages the new V row (the V page
// is dim-major: the new token is two bytes in every 32) for the consumer to
// patch in.  Every wave still issues at least PER / 2 copies of K and then
// PER / 2 of V for the chunk, and the staging copy comes before them, so the
// waits for a chunk's K and for its V still cover everything (they can only
// wait for one copy more than needed).
template <int D, int F>
__device__ __forceinline__ void issue_chunk(const DecodeArgs& a, uint32_t raw_id, uint8_t* buf, const Unit& x,
                                            bool last, uint8_t* stage, int32_t* newp, int wave, int lane) {
    using C = Cfg<D, F>;
    // an id outside the pool (a missing page or a stale plan) reads page 0
    const bool in_pool = raw_id < (uint32_t)a.num_pages;
    const int32_t phys = in_pool ? (int32_t)raw_id : 0;
    const int64_t blk = ((int64_t)phys * a.hkv + x.g) * C::PAGE;
    const uint8_t* kp = a.k_slab + blk;       // wave-uniform bases; per-lane 32-bit offsets
    const uint8_t* vp = a.v_slab + blk;
    const uint32_t kb = lds_addr_of(buf), vb = kb + C::PAGE;
    if constexpr (F == kFmtBF16) {
        if (a.append && last) {
            const int64_t nrow = ((int64_t)x.b * a.hkv + x.g) * D;     // the (b, g) row of k_new / v_new
            const int r = (x.hi - 1) & 15;                              // slot of position L - 1
            if (wave == 0) {
                if (lane < D / 8) dma16_s(a.v_new + nrow, (uint32_t)(lane * 16), lds_addr_of(stage));
                if (lane == 0) *newp = in_pool ? phys : -1;   // -1: the new row has no page to go to
            }
#pragma unroll
            for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
                const int inst = wave + kWaves * i;
                const int G = inst * 64 + lane;
                const int row = G / (C::ROW / 16), colp = G % (C::ROW / 16);
                if (row != r) dma16_s_nt(kp, (uint32_t)(row * C::ROW + (colp ^ (row & 15)) * 16), kb + inst * 1024);
            }
            // row r: ROW/16 granules, granule c landing at (c ^ (r & 15)); its
            // copy instruction(s) belong to wave (r / rows per 1 KiB) % 4
            constexpr int RPI = 1024 / C::ROW;                          // K rows per 1 KiB copy (1 or 2)
            if (wave == (r / RPI) % kWaves && lane < C::ROW / 16)
                dma16_s(a.k_new + nrow, (uint32_t)((lane ^ (r & 15)) * 16), kb + r * C::ROW);
#pragma unroll
            for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
                const int inst = wave + kWaves * i;
                const int gp = inst * 64 + lane, d = gp >> 1;
                dma16_s_nt(vp, (uint32_t)(d * 32 + (((gp & 1) ^ ((d >> 3) & 1)) * 16)), vb + inst * 1024);
            }
            return;
        }
    }
    // K: LDS granule G holds row G / (ROW/16), column (G % (ROW/16)) ^ (row & 15)
    // (LDS serves 16-byte reads 16 lanes at a time over 64 banks: the 16 rows
    // read at once land in 16 different bank groups)
#pragma unroll
    for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
        const int inst = wave + kWaves * i;
        const int G = inst * 64 + lane;
        const int row = G / (C::ROW / 16), colp = G % (C::ROW / 16);
        dma16_s_nt(kp, (uint32_t)(row * C::ROW + (colp ^ (row & 15)) * 16), kb + inst * 1024);
    }
    // V: the dim-major page block; for bf16 the two 16-byte halves of dim d
    // trade places when bit 3 of d is set, so that the 16 dims read at once
    // land in different bank groups
    if constexpr (C::HAS_V) {
#pragma unroll
        for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
            const int inst = wave + kWaves * i;
            if constexpr (!C::Q8) {
                const int gp = inst * 64 + lane, d = gp >> 1;
                dma16_s_nt(vp, (uint32_t)(d * 32 + (((gp & 1) ^ ((d >> 3) & 1)) * 16)), vb + inst * 1024);
            } else {
                dma16_s_nt(vp, (uint32_t)(inst * 1024 + lane * 16), vb + inst * 1024);
            }
        }
    }
    if constexpr (C::Q8) {
        // wave w copies 32 bytes of the page's 128 bytes of scales (k then v)
        if (lane < 2) {
            const int seg = wave * 2 + lane;                  // 16-byte piece 0..7
            const float* sb = (seg < 4) ? a.k_scale : a.v_scale;
            const float* src = sb + ((int64_t)phys * a.hkv + x.g) * kPage + (seg & 3) * 4;
            dma16(src, vb + C::PAGE + wave * 32);
        }
    }
}

// Partials cross workgroups, and for a unit spread over XCDs (whose L2s are
// not coherent with each other) they go through device-coherent accesses (the
// sc1 bit: agent-scope coherence), which need no writeback or invalidation of
// a whole L2; a unit on one XCD keeps them in that XCD's L2 (put4 / get4s
// with LOCAL).  They are issued in batches from inline assembly and awaited
// explicitly; the wait takes the loaded registers as operands, so nothing
// reads them earlier.
//
// Two hazards the compiler cannot see through this asm are handled by hand:
// - A store with more than 8 bytes of data reads its data registers after it
//   issues, so the next instruction must not overwrite them at once; put4
//   ends with an s_nop that keeps the next instruction out of that window.
// - A memory instruction that reads an MFMA result needs wait states after
//   the MFMA; mfma_settle() (24 wait states, more than any MFMA here needs)
//   separates the value product from the put4s that store its output.
__device__ __forceinline__ void mfma_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
// Partial exchange.  Device scope (sc1): the partials and the counter go
// through memory, for units whose workgroups sit on different XCDs.  Local:
// every workgroup of the unit is on one XCD, whose L2 all its CUs share, so
// stores stop in that L2 (the vector L1 writes through), the counter's atomic
// runs there, and loads skip only the L1 (sc0).
template <bool LOCAL>
__device__ __forceinline__ void put4(float* p, f32x4 v) {
    if constexpr (LOCAL) asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
    else asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}
template <bool LOCAL>
__device__ __forceinline__ void put2(float* p, float x, float y) {
    if constexpr (LOCAL) asm volatile("global_store_dwordx2 %0, %1, off" : : "v"(p), "v"(f32x2{x, y}) : "memory");
    else asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(f32x2{x, y}) : "memory");
}
// Scalar base + 32-bit byte offset forms: one address VGPR per partial
// serves all of a thread's items through the immediate offset.
template <bool LOCAL, int OFF>
__device__ __forceinline__ f32x4 get4s(const float* base, uint32_t voff) {
    f32x4 v;
    if constexpr (LOCAL)
        asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 sc0" : "=v"(v) : "v"(voff), "s"(base), "i"(OFF) : "memory");
    else
        asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 sc1" : "=v"(v) : "v"(voff), "s"(base), "i"(OFF) : "memory");
    return v;
}
template <bool LOCAL>
__device__ __forceinline__ f32x2 get2s(const float* base, uint32_t voff) {
    f32x2 v;
    if constexpr (LOCAL) asm volatile("global_load_dwordx2 %0, %1, %2 sc0" : "=v"(v) : "v"(voff), "s"(base) : "memory");
    else asm volatile("global_load_dwordx2 %0, %1, %2 sc1" : "=v"(v) : "v"(voff), "s"(base) : "memory");
    return v;
}
template <int N, typename T>
__device__ __forceinline__ void await(T (&regs)[N]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(regs[i]));
}

// Marks, when a workgroup starts a unit it shares with others inside one XCD,
// bit 16 + (its XCD) of the unit's counter word.  Issued at the unit's start,
// without waiting: the wait before the arrival (arrive_last) covers it long
// after it has landed, so it adds no round trip.
__device__ __forceinline__ void flag_xcd(uint32_t* counter, uint32_t xcc) {
    if (threadIdx.x == 0) {
        asm volatile("" : "+s"(xcc));   // form the flag here, not early in the kernel
        __hip_atomic_fetch_or(counter, 1u << (16 + xcc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Counts this workgroup's arrival at a unit and reports whether it was the
// last of `expected` (then every partial of the unit is complete).  The
// counter's low 16 bits count arrivals.  On the XCD-local path every
// workgroup of the unit set bit 16 + (its XCD) in the same word when it
// started the unit (flag_xcd), and the last to arrive checks that one bit is
// set in all: a unit whose workgroups ran on several XCDs exchanged its
// partials through L2s that do not see each other, so the merge may have read
// stale data, and the status word records it.  (A workgroup's flag is
// complete, vmcnt(0), before its arrival issues.)
template <bool LOCAL>
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* ticket, uint32_t xcc,
                                            uint32_t* status, bool check) {
    wait_vm<0>();               // this wave's partial stores (and its flag) are complete
    lds_barrier();              // ... and every wave's
    if (threadIdx.x == 0) {
        uint32_t old;
        if constexpr (LOCAL)
            old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
            old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *ticket = old;
        if (LOCAL && check && (old & 0xffffu) == expected - 1 && (old >> 16) != (1u << xcc))
            __hip_atomic_fetch_or(status, kStatusXcdSplit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_barrier();
    return (*ticket & 0xffffu) == expected - 1;
}

// One batch of a unit's merge: partial slots sl0, sl0 + G, ... (CNT of them,
// in workgroup order) folded into (M, L, acc).  All loads are issued before
// the first wait, and exactly CNT partials are read: the batch size is a
// template argument, so the last, partial batch of a unit neither loads
// padding nor holds registers whose definition depends on a branch (the loads
// are asynchronous, and a value merged from two branches could be copied
// before it lands).
template <int D, int CNT, bool LOCAL>
__device__ __forceinline__ void merge_batch(const float* o_base, const float* ml_base, uint32_t sl0, int32_t G,
                                            int d0, float& M, float& L, f32x4 (&acc)[D / 128]) {
    constexpr int IPT = D / 128;
    f32x2 ml[CNT];
    f32x4 ov[CNT * IPT];
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
        const uint32_t sl = sl0 + (uint32_t)(k * G);
        ml[k] = get2s<LOCAL>(ml_base, sl * 8u);
        const uint32_t ob = (sl * D + d0) * 4u;
        ov[k * IPT + 0] = get4s<LOCAL, 0>(o_base, ob);
        ov[k * IPT + 1] = get4s<LOCAL, 512>(o_base, ob);
        if constexpr (IPT > 2) {
            ov[k * IPT + 2] = get4s<LOCAL, 1024>(o_base, ob);
            ov[k * IPT + 3] = get4s<LOCAL, 1536>(o_base, ob);
        }
    }
    await(ml);
    await(ov);
    float Mb = M;
#pragma unroll
    for (int k = 0; k < CNT; ++k) Mb = fmaxf(Mb, ml[k].x);
    const float Mb_use = (Mb == -INFINITY) ? 0.0f : Mb;
    const float r = exp2f(M - Mb_use);            // rescale what came before
    L *= r;
#pragma unroll
    for (int j = 0; j < IPT; ++j) acc[j] *= r;
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
        const float wt = exp2f(ml[k].x - Mb_use);
        L += wt * ml[k].y;
#pragma unroll
        for (int j = 0; j < IPT; ++j) acc[j] += wt * ov[k * IPT + j];
    }
    M = Mb;
}

// Merges the partials of unit x (slots w + x.u for w in [w0, w1], in that
// order) and writes the G heads' bf16 outputs.  Thread t owns IPT = D/128
// 4-dim items of one head, dims 4 (t % 32) + 128 j, so one (m, l) pair per
// partial serves all of them while each load instruction still reads 512
// contiguous bytes per head; a pass covers 8 heads.  Partials go in batches
// of BATCH (all loads of a batch in flight together): the merging
// workgroup's own bandwidth bounds the merge, so the batches carry no
// padding.
template <int D, bool LOCAL>
__device__ __forceinline__ void merge_unit(const DecodeArgs& a, const Unit& x, int32_t w0, int32_t w1, int32_t G, int t) {
    constexpr int IPT = D / 128;
    constexpr int TPH = (D / 4) / IPT;                 // threads per head (32)
    constexpr int BATCH = (D == 512) ? 7 : 8;
    static_assert(IPT == 2 || IPT == 4, "items per thread");
    const int d0 = (t % TPH) * 4;
    // byte offsets below are 32-bit: the partial buffers are sized by the
    // host to (grid + units) * G * (D + 2) floats, far below 4 GiB
    const float* o_base = reinterpret_cast<const float*>(uniform_ptr(a.part_o));
    const float* ml_base = reinterpret_cast<const float*>(uniform_ptr(a.part_ml));
    for (int hb = 0; hb < G; hb += 256 / TPH) {
        const int hl = hb + t / TPH;
        if (hl >= G) continue;
        float M = -INFINITY, L = 0.f;
        f32x4 acc[IPT];
#pragma unroll
        for (int j = 0; j < IPT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (D == 256) {
            int32_t wb = w0;
            for (; wb + BATCH - 1 <= w1; wb += BATCH)
                merge_batch<D, BATCH, LOCAL>(o_base, ml_base, (uint32_t)((wb + x.u) * G + hl), G, d0, M, L, acc);
            const uint32_t sl0 = (uint32_t)((wb + x.u) * G + hl);
            switch (w1 - wb + 1) {    // the rest, 0 .. BATCH - 1 partials, without padding
                case 1: merge_batch<D, 1, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 2: merge_batch<D, 2, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 3: merge_batch<D, 3, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 4: merge_batch<D, 4, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 5: merge_batch<D, 5, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 6: merge_batch<D, 6, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                case 7: merge_batch<D, 7, LOCAL>(o_base, ml_base, sl0, G, d0, M, L, acc); break;
                default: break;
            }
        } else {
            // D = 512: one batch body for every batch, the last one padded by
            // re-reading slot w1 with weight zero (the exact-count form's extra
            // code cost this kernel more than the padding does)
            for (int32_t wb = w0; wb <= w1; wb += BATCH) {
                f32x2 ml[BATCH];
                f32x4 ov[BATCH * IPT];
#pragma unroll
                for (int k = 0; k < BATCH; ++k) {
                    const uint32_t sl = (uint32_t)((min(wb + k, w1) + x.u) * G + hl);
                    ml[k] = get2s<LOCAL>(ml_base, sl * 8u);
                    const uint32_t ob = (sl * D + d0) * 4u;
                    ov[k * IPT + 0] = get4s<LOCAL, 0>(o_base, ob);
                    ov[k * IPT + 1] = get4s<LOCAL, 512>(o_base, ob);
                    if constexpr (IPT > 2) {
                        ov[k * IPT + 2] = get4s<LOCAL, 1024>(o_base, ob);
                        ov[k * IPT + 3] = get4s<LOCAL, 1536>(o_base, ob);
                    }
                }
                await(ml);
                await(ov);
                float Mb = M;
#pragma unroll
                for (int k = 0; k < BATCH; ++k)
                    if (wb + k <= w1) Mb = fmaxf(Mb, ml[k].x);
                const float Mb_use = (Mb == -INFINITY) ? 0.0f : Mb;
                const float r = exp2f(M - Mb_use);            // rescale what came before
                L *= r;
#pragma unroll
                for (int j = 0; j < IPT; ++j) acc[j] *= r;
#pragma unroll
                for (int k = 0; k < BATCH; ++k) {
                    const float wt = (wb + k <= w1) ? exp2f(ml[k].x - Mb_use) : 0.0f;
                    L += wt * ml[k].y;
#pragma unroll
                    for (int j = 0; j < IPT; ++j) acc[j] += wt * ov[k * IPT + j];
                }
                M = Mb;
            }
        }
        const float inv = 1.0f / L;
        uint16_t* op = a.out + ((int64_t)x.b * a.hq + (int64_t)x.g * G + hl) * D + d0;
#pragma unroll
        for (int j = 0; j < IPT; ++j)
            *reinterpret_cast<u32x2*>(op + 128 * j) = u32x2{cvt_pk_bf16(acc[j][0] * inv, acc[j][1] * inv),
                                                          cvt_pk_bf16(acc[j][2] * inv, acc[j][3] * inv)};
    }
}

// int8 scores on fp16 MFMAs: a code c becomes the fp16 value c + 1152 (the
// byte c + 128 in the low mantissa byte of 1024.0: exact, two codes per byte
// permute, against a float conversion per code and a pack per pair for bf16).
// Q is scaled per wavefront by a power of two so that its largest |q| lies in
// [2^14, 2^15) (bf16 values there are fp16 values; an element more than 2^28
// below the largest becomes an fp16 subnormal, off by under 2^-24 after the
// scaling), the product q' (c + 1152) is exact
// in float32, and 1152 sum q' (the same fp16 values, summed in float32) is
// taken from each chunk's partial scores before the scale is undone: the
// offset never accumulates across chunks.  The value product stays bf16.
// int8 long-context full layer (8 x 131072 keys, D 512): 236 -> 215 us.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x4 i8x8_to_f16x8_off(u32x2 w) {
    const uint32_t a = w.x ^ 0x80808080u, b = w.y ^ 0x80808080u;
    return u32x4{__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u),
                 __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)};
}
__device__ __forceinline__ f32x4 mfma_16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}
// Q (bf16 pairs) -> fp16 pairs times 2^sh, sh chosen per wavefront so that
// the largest |q| lands in [2^14, 2^15); q_inv = 2^-sh; qoff = 1152 times
// the sum of the lane's head's fp16 values over the wavefront's dims.
template <int N>
__device__ __forceinline__ void q_to_f16(u32x4 (&qreg)[N], float& q_inv, float& qoff) {
    float am = 0.f;
#pragma unroll
    for (int kk = 0; kk < N; ++kk)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            am = fmaxf(am, fmaxf(fabsf(__uint_as_float(qreg[kk][w] << 16)),
                                 fabsf(__uint_as_float(qreg[kk][w] & 0xffff0000u))));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    am = wave_max_across_groups(am);
    const int e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(am));
    const int sh = min(126, max(-126, 15 - e));     // 2^sh and 2^-sh stay normal floats
    const float sc = __builtin_amdgcn_ldexpf(1.0f, sh);
    q_inv = __builtin_amdgcn_ldexpf(1.0f, -sh);
    float sum = 0.f;
#pragma unroll
    for (int kk = 0; kk < N; ++kk)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(qreg[kk][w] << 16) * sc,
                                                      __uint_as_float(qreg[kk][w] & 0xffff0000u) * sc);
            sum += (float)h[0] + (float)h[1];
            qreg[kk][w] = __builtin_bit_cast(uint32_t, h);
        }
    qoff = 1152.0f * wave_sum_across_groups(sum);
}

// Two 8-bit codes of a word -> a bf16 pair (exact), for the 8-bit formats.
template <int F>
__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t word, int byte_lo) {
    if constexpr (F == kFmtFP8) return fp8x2_to_bf16x2(word, byte_lo);
    else return i8x2_to_bf16x2(word, byte_lo);
}

template <int D, int F>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a) {
    using C = Cfg<D, F>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    __shared__ uint32_t ticket;
    f32x4* sx = reinterpret_cast<f32x4*>(lds + C::NBUF * C::BUF);
    int32_t* seq_lds = reinterpret_cast<int32_t*>(lds + C::NBUF * C::BUF + C::SX);
    const SeqTable st{seq_lds, seq_lds + pakv::kDecodeMaxSeqs + 1};
    uint8_t* stage = lds + C::NBUF * C::BUF + C::SX + C::SEQ;
    int32_t* newp = reinterpret_cast<int32_t*>(stage + C::NBUF * C::STAGE);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int qg = lane >> 4;            // 4-row group of the MFMA layouts
    const int col = lane & 15;           // head column
    const int32_t G = a.group;
    const int32_t B = a.num_seqs;
    const int32_t U = B * a.hkv;
    uint32_t xcc;                        // the XCD this workgroup runs on
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 15u;

    // the schedule: the sequence table into LDS, this workgroup's record and
    // the page ids of its first 64 chunks, all loads issued before any wait
    // (one round trip); then Q of the first unit and the first chunks' copies
    // (a second round trip, awaited with the first chunk)
    // the plan wrote this workgroup's record at its own index: workgroups go
    // to the XCDs in turn (blockIdx mod 8), and the plan gave each XCD a
    // contiguous block of its runs, so a unit's runs mostly share one XCD's L2
    const int32_t xblk = (a.grid & 7) == 0 ? a.grid >> 3 : 0;
    const int32_t* rec = a.sched + a.s_rec + (int64_t)blockIdx.x * pakv::kPlanRecord;
    int32_t tab_o[4], tab_l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {        // B <= 1023: at most four entries per thread
        const int i = threadIdx.x + 256 * k;
        tab_o[k] = (i <= B) ? a.sched[a.s_soff + i] : 0;
        tab_l[k] = (i < B) ? a.sched[a.s_slen + i] : 1;
    }
    const int32_t field = rec[min(lane, 15)];
    const int32_t hdr = a.sched[min(lane, 7)];     // the plan's header
    uint32_t ids = (uint32_t)rec[pakv::kPlanRecIds + lane];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = threadIdx.x + 256 * k;
        if (i <= B) st.soff[i] = tab_o[k];
        if (i < B) st.slen[i] = clamp_i32(tab_l[k], 1, a.max_kv_len);
    }
    const int32_t c_begin = max(__builtin_amdgcn_readlane(field, 0), 0);
    const int32_t c_end = (int32_t)min((int64_t)__builtin_amdgcn_readlane(field, 1), a.s_cap);
    const int32_t u_first = clamp_i32(__builtin_amdgcn_readlane(field, 2), 0, U - 1);
    const int32_t kc_first = max(__builtin_amdgcn_readlane(field, 3), 0);
    // stream-K runs (per > 0) or unit-aligned runs (per = 0; the unit's
    // workgroups are [rw0, rw1], clamped so that a stale plan stays in bounds)
    const int32_t per = max(__builtin_amdgcn_readlane(field, 4), 0);
    // the run's number in the plan (it names the run's partial slots)
    const int32_t vb = clamp_i32(__builtin_amdgcn_readlane(field, 7), 0, a.grid - 1);
    const int32_t rw0 = clamp_i32(__builtin_amdgcn_readlane(field, 5), 0, vb);
    const int32_t rw1 = clamp_i32(__builtin_amdgcn_readlane(field, 6), vb, a.grid - 1);
    const bool rec_local = __builtin_amdgcn_readlane(field, 8) != 0;
    __syncthreads();
    // a plan made for another shape (sequences, Hkv, window, length bound or
    // grid) describes another split: every workgroup returns before touching
    // a counter or an output, and the status word says why
    {
        const bool same = __builtin_amdgcn_readlane(hdr, 0) == pakv::kPlanMagic &&
                          __builtin_amdgcn_readlane(hdr, 3) == a.grid && __builtin_amdgcn_readlane(hdr, 4) == B &&
                          __builtin_amdgcn_readlane(hdr, 5) == a.hkv && __builtin_amdgcn_readlane(hdr, 6) == a.window &&
                          __builtin_amdgcn_readlane(hdr, 7) == a.max_kv_len;
        if (!same) {
            if (blockIdx.x == 0 && threadIdx.x == 0)
                __hip_atomic_fetch_or(a.status, kStatusPlanMismatch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
    if (c_begin >= c_end) return;
    const int32_t total = c_end - c_begin;

    Unit uc = unit_of(a, st, u_first);
    int32_t kc = min(kc_first, uc.n - 1);
    // the workgroups [w0, w1] of a unit: from the stream-K run length, or the
    // aligned split's record (one unit per workgroup there)
    auto unit_span = [&](const Unit& x, int32_t& w0, int32_t& w1) {
        w0 = per > 0 ? x.first / per : rw0;
        w1 = per > 0 ? (x.first + x.n - 1) / per : rw1;
    };
    // a unit whose runs all lie in one XCD's block merges in that XCD's L2:
    // stream-K blocks are grid / 8 runs; the aligned split's record says so
    auto is_local = [&](int32_t w0, int32_t w1) {
        return per > 0 ? (xblk > 0 && w0 / xblk == w1 / xblk) : rec_local;
    };
    auto flag_if_local = [&](const Unit& x) {
        int32_t w0, w1;
        unit_span(x, w0, w1);
        if (a.check_xcd && w0 != w1 && is_local(w0, w1)) flag_xcd(a.arrivals + x.u, xcc);
    };
    flag_if_local(uc);
    Unit ui = uc;                                 // issue cursor
    int32_t ki = kc;
    const int dq = wave * (D / 4);
    u32x4 qreg[C::KK];
    float q_inv = 1.f, qoff = 0.f;                // int8: Q's scale back, and 1152 sum q'
    load_q<D>(a, uc, G, col, qg, dq, qreg);       // complete once chunk 0's copies are
#pragma unroll
    for (int c = 0; c < C::NBUF - 1; ++c) {
        if (c < total) {
            issue_chunk<D, F>(a, (uint32_t)__builtin_amdgcn_readlane(ids, c), lds + c * C::BUF, ui,
                                 ki == ui.n - 1, stage + c * C::STAGE, newp + c, wave, lane);
            advance(a, st, U, ui, ki);
        }
    }

    f32x4 o[C::MT];
#pragma unroll
    for (int m = 0; m < C::MT; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int32_t i = 0; i < total; ++i) {
        // bf16: this chunk's K only (each wave issues K before V); its V is
        // awaited after the scores, so the score product overlaps V's arrival
        // (with one chunk ahead, only this chunk's copies are in flight here).
        // K=V: the chunk's copies are all K.
        static_assert(C::Q8 || C::NBUF == 2, "the split K / V waits count one chunk in flight");
        if constexpr (F == kFmtBF16) wait_vm<C::PER / 2>();
        else if constexpr (F == kFmtKEQV) wait_vm<0>();
        else wait_chunks<C::PER, C::NBUF>(min(C::NBUF - 2, total - 1 - i));
        lds_barrier();
        if (kc == 0 || i == 0) {
            // a new unit: its Q.  The first was issued before chunk 0's copies,
            // so the wait above covered it; a later one was issued when the
            // previous unit ended, after the copies in flight, and this wait
            // drains them too, but only here, once per unit.
            if (i > 0) wait_vm<0>();
            take_q(qreg, col < G);
            if constexpr (F == kFmtINT8) q_to_f16(qreg, q_inv, qoff);
        }
        {
            const int32_t j = i + C::NBUF - 1;        // chunk to copy now
            if (j < total) {
                if ((j & 63) == 0) {                  // next window of page ids (drains, once per 64)
                    ids = sched_ids(a, c_begin + j, min(total - j, 64), lane);
                    wait_vm<0>();
                }
                issue_chunk<D, F>(a, (uint32_t)__builtin_amdgcn_readlane(ids, j & 63),
                                     lds + (j % C::NBUF) * C::BUF, ui, ki == ui.n - 1,
                                     stage + (j % C::NBUF) * C::STAGE, newp + (j % C::NBUF), wave, lane);
                advance(a, st, U, ui, ki);
            }
        }
        const uint8_t* kbuf = lds + (i % C::NBUF) * C::BUF;
        const uint8_t* vbuf = kbuf + C::PAGE;
        const int32_t t0 = (uc.page0 + kc) * kChunk;
        if constexpr (F == kFmtBF16) {
            if (a.append && kc == uc.n - 1) {
                // the new token (slot r of this page): write its K row (already
                // in LDS, from k_new) and its staged V values to the slab; the V
                // values are patched into the staged page once its copies have
                // landed (after the score exchange)
                // (a position whose page id lies outside the pool is not
                // written, as the store drops such rows; it is still attended)
                const int r = (uc.hi - 1) & 15;
                const uint8_t* sg = stage + (i % C::NBUF) * C::STAGE;
                const int32_t np = newp[i % C::NBUF];
                if (np >= 0) {
                    const int64_t blk = ((int64_t)np * a.hkv + uc.g) * C::PAGE;
                    uint8_t* kdst = const_cast<uint8_t*>(a.k_slab) + blk + r * C::ROW;
                    uint8_t* vdst = const_cast<uint8_t*>(a.v_slab) + blk + r * 2;
                    for (int d = threadIdx.x; d < D; d += 256)
                        *reinterpret_cast<uint16_t*>(vdst + d * 32) = *reinterpret_cast<const uint16_t*>(sg + 2 * d);
                    if (threadIdx.x < C::ROW / 16) {
                        const int c = threadIdx.x;
                        *reinterpret_cast<u32x4*>(kdst + c * 16) =
                            *reinterpret_cast<const u32x4*>(kbuf + r * C::ROW + ((c ^ (r & 15)) * 16));
                    }
                }
            }
        }

        // ---- partial scores over this wave's dim quarter --------------------
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;     // K=V: this lane's part of the key row's sum of squares
        {
            const int row = col;
            const uint8_t* krow = kbuf + row * C::ROW;
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) {
                const int e0 = dq + 32 * kk + 8 * qg;          // first of 8 dims
                u32x4 ka;
                if constexpr (!C::Q8) {
                    ka = *reinterpret_cast<const u32x4*>(krow + (((e0 >> 3) ^ (row & 15)) * 16));
                    if constexpr (F == kFmtKEQV) {
                        // one dot2 per pair (v_dot2c_f32_bf16: exact products,
                        // float32 sum) instead of two unpacks and two FMAs: the
                        // K=V layers of the 26B-like step ~3% faster
#pragma unroll
                        for (int w = 0; w < 4; ++w) ss = sq_sum_bf16x2(ka[w], ss);
                    }
                } else {
                    const u32x2 w = *reinterpret_cast<const u32x2*>(krow + (((e0 >> 4) ^ (row & 15)) * 16) + (e0 & 8));
                    if constexpr (F == kFmtINT8) ka = i8x8_to_f16x8_off(w);
                    else ka = u32x4{codes_to_bf16x2<F>(w.x, 0), codes_to_bf16x2<F>(w.x, 2),
                                    codes_to_bf16x2<F>(w.y, 0), codes_to_bf16x2<F>(w.y, 2)};
                }
                if constexpr (F == kFmtINT8) acc = mfma_16x16x32_f16(ka, qreg[kk], acc);
                else acc = mfma_16x16x32(ka, qreg[kk], acc);
            }
            if constexpr (F == kFmtINT8) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = (acc[e] - qoff) * q_inv;
            }
        }
        float* ssx = reinterpret_cast<float*>(sx + kWaves * 64);   // K=V: [wave][16 rows]
        if constexpr (F == kFmtKEQV) {
            // the four 16-lane rows hold four dim groups of key row `col`
            ss = wave_sum_across_groups(ss);
            if (qg == 0) ssx[wave * 16 + col] = ss;
        }
        if constexpr (F == kFmtBF16) {
            // this chunk's V: past it, only the next chunk's copies (issued at
            // the top of this step) may still be in flight
            if (i + 1 < total) wait_vm<C::PER>();
            else wait_vm<0>();
        }
        sx[wave * 64 + lane] = acc;
        lds_barrier();
        if constexpr (F == kFmtBF16) {
            if (a.append && kc == uc.n - 1) {
                // every wave's V copies have landed: patch in the new token's V
                // (two bytes per dim, each dim's 32 bytes copied by one wave)
                const int r = (uc.hi - 1) & 15;
                const uint8_t* sg = stage + (i % C::NBUF) * C::STAGE;
                uint8_t* vpatch = lds + (i % C::NBUF) * C::BUF + C::PAGE;
                for (int d = threadIdx.x; d < D; d += 256)
                    *reinterpret_cast<uint16_t*>(vpatch + d * 32 + ((((r >> 3) ^ (d >> 3)) & 1) << 4) + (r & 7) * 2) =
                        *reinterpret_cast<const uint16_t*>(sg + 2 * d);
                lds_barrier();
            }
        }
        f32x4 tot = sx[lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) tot += sx[w * 64 + lane];

        // ---- online softmax: lane holds tokens t0 + 4*qg + i -----------------
        float ks[4] = {1.f, 1.f, 1.f, 1.f}, vs[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (C::Q8) {
            const float* scl = reinterpret_cast<const float*>(vbuf + C::PAGE);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[e] = scl[4 * qg + e];
                vs[e] = scl[16 + 4 * qg + e];
            }
        }
        if constexpr (F == kFmtKEQV) {
            // value row = key row / sqrt(mean square + eps): the factor goes
            // into the weights, the key row itself into the value product
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * qg + e;
                float t = ssx[r];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) t += ssx[w * 16 + r];
                vs[e] = __builtin_amdgcn_rsqf(t * (1.0f / D) + a.v_norm_eps);
            }
        }
        float sc[4];
        bool valid[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int32_t t = t0 + 4 * qg + e;
            valid[e] = (t >= uc.lo) && (t < uc.hi);
            float v = tot[e] * a.score_scale;
            if constexpr (C::Q8) v *= ks[e];
            sc[e] = valid[e] ? v : -INFINITY;
            mx = fmaxf(mx, sc[e]);
        }
        mx = wave_max_across_groups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        // v_exp_f32 directly: a weight below 2^-126 of the row's largest
        // becomes zero instead of a denormal
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float p[4], psum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
            psum += p[e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = p[e];
            if constexpr (F != kFmtBF16) x *= vs[e];
            pv[e] = valid[e] ? x : 0.0f;
        }
        const u32x2 pb = u32x2{cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3])};
        const bool full = (t0 >= uc.lo) && (t0 + kChunk <= uc.hi);

        // ---- values: this wave's quarter of the output dims ------------------
#pragma unroll
        for (int m = 0; m < C::MT; ++m) {
            const int d = dq + 16 * m + col;
            u32x2 va;
            if constexpr (F == kFmtBF16) {
                va = *reinterpret_cast<const u32x2*>(vbuf + d * 32 + ((((qg >> 1) ^ (d >> 3)) & 1) << 4) + 8 * (qg & 1));
            } else if constexpr (F == kFmtKEQV) {
                // the value operand (one dim, four tokens) from the key rows,
                // with one transposing read: lane j of 16-lane group qg
                // addresses key row 4 qg + j / 4, dims dq + 16 m + 4 (j % 4)
                // .. + 3 (in granule dim / 8 ^ row), and receives tokens
                // 4 qg .. + 3 of dim dq + 16 m + col
                const int r = 4 * qg + (col >> 2);
                const int dd = dq + 16 * m + 4 * (col & 3);
                va = lds_read_tr16(kbuf + r * C::ROW + ((((dd >> 3) ^ r) & (C::ROW / 16 - 1)) << 4) + (dd & 7) * 2);
            } else {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(vbuf + d * 16 + 4 * qg);
                va = u32x2{codes_to_bf16x2<F>(w, 0), codes_to_bf16x2<F>(w, 2)};
            }
            // slots outside the visible range may hold NaN (int8 codes cannot)
            if (F != kFmtINT8 && !full) {
                va.x &= (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
                va.y &= (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
            }
            o[m] = o[m] * alpha;
            o[m] = mfma_16x16x16(va, pb, o[m]);
        }

        // ---- end of this run's part of the unit --------------------------------
        if (kc == uc.n - 1 || i == total - 1) {
            const float l_tot = wave_sum_across_groups(l_run);
            int32_t w0, w1;
            unit_span(uc, w0, w1);
            if (w0 == w1) {
                // the whole unit is in this run: normalise and write the outputs
                if (col < G) {
                    const float inv = 1.0f / l_tot;
                    uint16_t* op = a.out + ((int64_t)uc.b * a.hq + (int64_t)uc.g * G + col) * D + dq;
#pragma unroll
                    for (int m = 0; m < C::MT; ++m)
                        *reinterpret_cast<u32x2*>(op + 16 * m + 4 * qg) =
                            u32x2{cvt_pk_bf16(o[m][0] * inv, o[m][1] * inv), cvt_pk_bf16(o[m][2] * inv, o[m][3] * inv)};
                }
            } else {
                const int64_t slot = ((int64_t)vb + uc.u) * G;
                // every run of the unit on one XCD (the check needs no
                // communication: the split and the numbering are fixed)
                const bool local = is_local(w0, w1);
                mfma_settle();
                if (local) {
                    if (col < G) {
                        float* po = a.part_o + (slot + col) * D + dq;
#pragma unroll
                        for (int m = 0; m < C::MT; ++m) put4<true>(po + 16 * m + 4 * qg, o[m]);
                        if (wave == 0 && qg == 0) put2<true>(a.part_ml + (slot + col) * 2, m_run, l_tot);
                    }
                    // the last of the unit's partials to arrive merges them all
                    if (arrive_last<true>(a.arrivals + uc.u, (uint32_t)(w1 - w0 + 1), &ticket, xcc, a.status,
                                          a.check_xcd != 0)) {
                        merge_unit<D, true>(a, uc, w0, w1, G, threadIdx.x);
                        if (threadIdx.x == 0)
                            __hip_atomic_store(a.arrivals + uc.u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                } else {
                    if (col < G) {
                        float* po = a.part_o + (slot + col) * D + dq;
#pragma unroll
                        for (int m = 0; m < C::MT; ++m) put4<false>(po + 16 * m + 4 * qg, o[m]);
                        if (wave == 0 && qg == 0) put2<false>(a.part_ml + (slot + col) * 2, m_run, l_tot);
                    }
                    if (arrive_last<false>(a.arrivals + uc.u, (uint32_t)(w1 - w0 + 1), &ticket, xcc, a.status,
                                          false)) {
                        merge_unit<D, false>(a, uc, w0, w1, G, threadIdx.x);
                        if (threadIdx.x == 0)
                            __hip_atomic_store(a.arrivals + uc.u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
        }
        // a unit ends: the next one's Q, and its accumulators start empty (set
        // here rather than at its first chunk, so that neither o nor Q is live
        // across the merge above)
        const bool ended = (kc == uc.n - 1);
        advance(a, st, U, uc, kc);
        if (ended && i + 1 < total) {
            flag_if_local(uc);
            load_q<D>(a, uc, G, col, qg, dq, qreg);
#pragma unroll
            for (int m = 0; m < C::MT; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            l_run = 0.0f;
        }
    }
    wait_vm<0>();
}

// Writes the XCD each workgroup runs on (the hardware XCC id).
__global__ __launch_bounds__(64) void xcd_probe_kernel(int32_t* out, int32_t n) {
    uint32_t id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    if (threadIdx.x == 0 && (int32_t)blockIdx.x < n) out[blockIdx.x] = (int32_t)(id & 0xfu);
}

}  // namespace

namespace pakv {

// The workspace of pakv_paged_attn_decode_noalloc, for callers that cannot
// allocate: one copy per GPU, held until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in); it takes
// the device address from hipGetSymbolAddress, once per device.
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

int noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static void* per_device[kNoallocMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kNoallocMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // with `dev` current
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return 0;
}

int launch_xcd_probe(int32_t* out, int32_t n, void* stream) {
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(n), dim3(64), 0, static_cast<hipStream_t>(stream), out, n);
    return (int)hipGetLastError();
}

static DecodeArgs args_of(const DecodeLaunch& s) {
    DecodeArgs a;
    a.k_slab = static_cast<const uint8_t*>(s.slab.k);
    a.v_slab = static_cast<const uint8_t*>(s.slab.v);
    a.k_scale = s.slab.k_scale;
    a.v_scale = s.slab.v_scale;
    a.num_pages = s.slab.num_pages;
    a.max_pages = s.max_pages;
    a.q = s.q;
    a.out = s.out;
    a.num_seqs = s.num_seqs;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.group = s.plan.group;
    a.window = s.window;
    a.score_scale = s.sm_scale * kLog2e;
    a.max_kv_len = s.max_kv_len;
    a.grid = s.plan.grid;
    a.sched = s.sched;
    a.s_soff = s.layout.soff;
    a.s_slen = s.layout.slen;
    a.s_rec = s.layout.rec;
    a.s_ids = s.layout.ids;
    a.s_cap = s.layout.cap;
    a.status = s.status;
    a.arrivals = s.arrivals;
    a.part_o = s.part_o;
    a.part_ml = s.part_ml;
    a.k_new = s.k_new;
    a.v_new = s.v_new;
    a.append = s.append;
    a.zero_arrivals = s.zero_arrivals;
    a.v_norm_eps = s.v_norm_eps;
    a.check_xcd = s.check_xcd;
    a.bad_ids = debug_bad_ids_ptr();
    return a;
}

int launch_decode_plan(const DecodeLaunch& s, void* stream) {
    const DecodeArgs a = args_of(s);
    hipLaunchKernelGGL(decode_plan_kernel, dim3(s.plan.grid), dim3(256), 0, static_cast<hipStream_t>(stream), a,
                       s.page_table, s.kv_lens);
    return (int)hipGetLastError();
}

int launch_decode_plan2(const DecodeLaunch& s0, const DecodeLaunch& s1, void* stream) {
    const DecodeArgs a0 = args_of(s0), a1 = args_of(s1);
    hipLaunchKernelGGL(decode_plan2_kernel, dim3(s0.plan.grid + s1.plan.grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a0, a1, s0.page_table, s1.page_table, s0.kv_lens);
    return (int)hipGetLastError();
}

int launch_decode(const DecodeLaunch& s, void* stream) {
    const DecodeArgs a = args_of(s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid1(s.plan.grid);
    const int f = s.k_eq_v ? kFmtKEQV
                           : (s.kv_dtype == PAKV_KV_INT8_PTH ? kFmtINT8 : (s.kv_dtype == PAKV_KV_FP8_PTH ? kFmtFP8 : kFmtBF16));
    const int K = PAKV_TIME_DECODE;
    const dim3 blk(256);
    if (s.head_dim == 256) {
        switch (f) {
            case kFmtINT8: launch(K, decode_kernel<256, kFmtINT8>, grid1, blk, 0, st, a); break;
            case kFmtFP8: launch(K, decode_kernel<256, kFmtFP8>, grid1, blk, 0, st, a); break;
            case kFmtKEQV: launch(K, decode_kernel<256, kFmtKEQV>, grid1, blk, 0, st, a); break;
            default: launch(K, decode_kernel<256, kFmtBF16>, grid1, blk, 0, st, a); break;
        }
    } else {
        switch (f) {
            case kFmtINT8: launch(K, decode_kernel<512, kFmtINT8>, grid1, blk, 0, st, a); break;
            case kFmtFP8: launch(K, decode_kernel<512, kFmtFP8>, grid1, blk, 0, st, a); break;
            case kFmtKEQV: launch(K, decode_kernel<512, kFmtKEQV>, grid1, blk, 0, st, a); break;
            default: launch(K, decode_kernel<512, kFmtBF16>, grid1, blk, 0, st, a); break;
        }
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
