// paged_attn_decode: split-KV decode with a deterministic combine.
//
// Pass 1 (partial), stream-K: the work of all (sequence b, KV head g) units
// is a stream of 16-token chunks (one page each): unit (b, g) covers the
// pages that hold its visible keys [lo, L).  A fixed grid of kGrid persistent
// workgroups (4 wavefronts each) takes equal, contiguous runs of that stream,
// so every workgroup moves the same number of bytes whatever the length mix.
// A run that crosses unit boundaries produces one partial (o, m, l) per unit
// it touches, stored at slot (workgroup + unit).  Chunks are streamed into
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
// partials in workgroup order: M = max_s m_s,
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

#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 16;        // tokens per staged chunk (one page)

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
    uint32_t* arrivals;     // [U] partials written per unit; zero between calls
    float* part_o;          // [grid + U][G][D]
    float* part_ml;         // [grid + U][G][2]
};

// ---- asynchronous global -> LDS copies -----------------------------------
// One instruction copies 16 bytes per active lane; lane i writes LDS byte
// address m0 + 16*i.  M0 is saved and restored around it (the compiler keeps
// its own values there), with the one wait state the hardware needs between
// writing M0 and an LDS-DMA instruction.  The compiler does not track these
// copies: completion is awaited explicitly (wait_vm) before a barrier.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gaddr)
        : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Waits for this wave's copies so that at most `newer` chunks' copies stay in
// flight (newer <= NBUF - 2).
template <int PER, int NBUF>
__device__ __forceinline__ void wait_chunks(int newer) {
    if constexpr (NBUF >= 5) { if (newer >= 3) { wait_vm<3 * PER>(); return; } }
    if constexpr (NBUF >= 4) { if (newer >= 2) { wait_vm<2 * PER>(); return; } }
    if constexpr (NBUF >= 3) { if (newer >= 1) { wait_vm<PER>(); return; } }
    wait_vm<0>();
}

// Barrier for LDS traffic only: waits for this wave's LDS reads/writes (not
// for the global->LDS copies in flight) and orders the compiler around it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) { return (uint32_t)(uintptr_t)p; }

template <int D, bool INT8>
struct Cfg {
    static constexpr int ES = INT8 ? 1 : 2;                 // bytes per code
    static constexpr int ROW = D * ES;                      // bytes per K row
    static constexpr int PAGE = 16 * D * ES;                // bytes per (page, head) block
    static constexpr int SCALE_BYTES = INT8 ? 128 : 0;      // k and v scales of one page
    static constexpr int BUF = 2 * PAGE + SCALE_BYTES;
    static constexpr int NBUF = (D == 512 && !INT8) ? 2 : 4;
    static constexpr int KV_DMA = 2 * PAGE / (1024 * kWaves);   // copies per wave per chunk
    static constexpr int PER = KV_DMA + (INT8 ? 1 : 0);
    static constexpr int SX = kWaves * 64 * 16;             // partial-score exchange
    static constexpr int OFF = ((pakv::kDecodeMaxUnits + 1) * 4 + 15) & ~15;
    static constexpr int LDS = NBUF * BUF + SX + OFF;
    static constexpr int KK = D / 128;                      // 32-dim steps in a wave's quarter
    static constexpr int MT = D / 64;                       // 16-dim output tiles in a quarter
    static_assert(LDS <= 80 * 1024, "two workgroups per CU");
};

// Chunks of a unit: pages from lo/16 to (L-1)/16.
struct Unit {
    int32_t u, b, g, lo, hi, page0, n;
};

__device__ __forceinline__ Unit make_unit(const DecodeArgs& a, const int32_t* __restrict__ kv_lens, int32_t u) {
    Unit x;
    x.u = u;
    x.b = u / a.hkv;
    x.g = u - x.b * a.hkv;
    const int32_t len = clamp_i32(kv_lens[x.b], 1, a.max_kv_len);
    x.hi = len;
    x.lo = (a.window > 0 && len > a.window) ? len - a.window : 0;
    x.page0 = x.lo >> 4;
    x.n = ((len + 15) >> 4) - x.page0;
    return x;
}

// off[u] = first chunk of unit u in the stream, off[U] = total (block-wide scan).
__device__ __forceinline__ void build_offsets(const DecodeArgs& a, const int32_t* __restrict__ kv_lens,
                                              int32_t* off, int32_t U) {
    __shared__ int32_t wave_tot[kWaves];
    const int t = threadIdx.x;
    const int per_t = (U + 255) / 256;
    const int u0 = t * per_t, u1 = min(u0 + per_t, U);
    int32_t local = 0;
    for (int u = u0; u < u1; ++u) local += make_unit(a, kv_lens, u).n;
    // inclusive scan of `local` across the block
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
    int32_t run = before + incl - local;     // exclusive prefix of this thread's units
    for (int u = u0; u < u1; ++u) {
        off[u] = run;
        run += make_unit(a, kv_lens, u).n;
    }
    if (t == 255) off[U] = before + incl;
    __syncthreads();
}

template <int D, bool INT8>
__device__ __forceinline__ void issue_chunk(const DecodeArgs& a, const int32_t* __restrict__ page_table,
                                            uint8_t* buf, const Unit& x, int32_t k, int wave, int lane) {
    using C = Cfg<D, INT8>;
    int32_t phys = page_table[(int64_t)x.b * a.max_pages + x.page0 + k];
    phys = ((uint32_t)phys < (uint32_t)a.num_pages) ? phys : 0;   // out-of-pool ids never fault
    const int64_t blk = ((int64_t)phys * a.hkv + x.g) * C::PAGE;
    const uint8_t* kp = a.k_slab + blk;
    const uint8_t* vp = a.v_slab + blk;
    const uint32_t kb = lds_addr_of(buf), vb = kb + C::PAGE;
    // K: LDS granule G holds row G / (ROW/16), column (G % (ROW/16)) ^ (row & 7)
#pragma unroll
    for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
        const int inst = wave + kWaves * i;
        const int G = inst * 64 + lane;
        const int row = G / (C::ROW / 16), colp = G % (C::ROW / 16);
        dma16(kp + row * C::ROW + (colp ^ (row & 7)) * 16, kb + inst * 1024);
    }
    // V: the dim-major page block, copied as is
#pragma unroll
    for (int i = 0; i < C::PAGE / 1024 / kWaves; ++i) {
        const int inst = wave + kWaves * i;
        dma16(vp + inst * 1024 + lane * 16, vb + inst * 1024);
    }
    if constexpr (INT8) {
        // wave w copies 32 bytes of the page's 128 bytes of scales (k then v)
        if (lane < 2) {
            const int seg = wave * 2 + lane;                  // 16-byte piece 0..7
            const float* sb = (seg < 4) ? a.k_scale : a.v_scale;
            const float* src = sb + ((int64_t)phys * a.hkv + x.g) * kPage + (seg & 3) * 4;
            dma16(src, vb + C::PAGE + wave * 32);
        }
    }
}

// Q^T operand of a wave's dim quarter: column `col` = head g*G + col (zero
// for padding columns), dims dq + 32*kk + 8*qg .. +8.
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, const Unit& x, int32_t G, int col, int qg, int dq,
                                       u32x4 (&qreg)[D / 128]) {
    const bool real = col < G;
    const uint16_t* qp = a.q + ((int64_t)x.b * a.hq + (int64_t)x.g * G + (real ? col : 0)) * D + dq + 8 * qg;
#pragma unroll
    for (int kk = 0; kk < D / 128; ++kk)
        qreg[kk] = real ? *reinterpret_cast<const u32x4*>(qp + 32 * kk) : u32x4{0, 0, 0, 0};
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other) through device-coherent accesses (the sc1 bit: agent-scope
// coherence), which need no writeback or invalidation of a whole L2.  They are
// issued in batches from inline assembly and awaited explicitly; the wait
// takes the loaded registers as operands, so nothing reads them earlier.
__device__ __forceinline__ void put4(float* p, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void put2(float* p, float x, float y) {
    asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(f32x2{x, y}) : "memory");
}
__device__ __forceinline__ f32x4 get4(const float* p) {
    f32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
    return v;
}
__device__ __forceinline__ f32x2 get2(const float* p) {
    f32x2 v;
    asm volatile("global_load_dwordx2 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
    return v;
}
template <int N, typename T>
__device__ __forceinline__ void await(T (&regs)[N]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(regs[i]));
}

// Counts this workgroup's arrival at a unit and reports whether it was the
// last of `expected` (then every partial of the unit is complete).
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* ticket) {
    wait_vm<0>();               // this wave's partial stores are complete
    lds_barrier();              // ... and every wave's
    if (threadIdx.x == 0)
        *ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    return *ticket == expected - 1;
}

// Merges the partials of unit x (slots w + x.u for w in [w0, w1], in that
// order) and writes the G heads' bf16 outputs.  64 threads per head, each
// owning D/64 dims; partials are read 8 slots per batch.
template <int D>
__device__ void merge_unit(const DecodeArgs& a, const Unit& x, int32_t w0, int32_t w1, int32_t G, int t) {
    constexpr int DPT = D / 64;
    constexpr int NV = DPT / 4;
    constexpr int BATCH = 8;
    for (int hl = t >> 6; hl < G; hl += kWaves) {
        const int d0 = (t & 63) * DPT;
        // running max and rescaled sums over batches, in slot order
        float M = -INFINITY, L = 0.f;
        f32x4 acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t wb = w0; wb <= w1; wb += BATCH) {
            f32x2 ml[BATCH];
            f32x4 ov[BATCH * NV];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int32_t w = min(wb + k, w1);
                const int64_t sl = ((int64_t)w + x.u) * G + hl;
                ml[k] = get2(a.part_ml + sl * 2);
#pragma unroll
                for (int v = 0; v < NV; ++v) ov[k * NV + v] = get4(a.part_o + sl * D + d0 + 4 * v);
            }
            await(ml);
            await(ov);
            float Mb = M;
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                if (wb + k <= w1) Mb = fmaxf(Mb, ml[k].x);
            const float Mb_use = (Mb == -INFINITY) ? 0.0f : Mb;
            const float r = exp2f(M - Mb_use);         // rescale what came before
            L *= r;
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[v] *= r;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                if (wb + k > w1) break;
                const float wt = exp2f(ml[k].x - Mb_use);
                L += wt * ml[k].y;
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] += wt * ov[k * NV + v];
            }
            M = Mb;
        }
        const float inv = 1.0f / L;
        uint16_t* op = a.out + ((int64_t)x.b * a.hq + (int64_t)x.g * G + hl) * D + d0;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            *reinterpret_cast<u32x2*>(op + 4 * v) =
                u32x2{pack_bf16x2(acc[v][0] * inv, acc[v][1] * inv), pack_bf16x2(acc[v][2] * inv, acc[v][3] * inv)};
    }
}

template <int D, bool INT8>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a, const int32_t* __restrict__ page_table,
                                                                 const int32_t* __restrict__ kv_lens) {
    using C = Cfg<D, INT8>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    int32_t* off = reinterpret_cast<int32_t*>(lds + C::NBUF * C::BUF + C::SX);
    __shared__ uint32_t ticket;
    f32x4* sx = reinterpret_cast<f32x4*>(lds + C::NBUF * C::BUF);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int qg = lane >> 4;            // 4-row group of the MFMA layouts
    const int col = lane & 15;           // head column
    const int32_t G = a.group;
    const int32_t U = a.num_seqs * a.hkv;

    build_offsets(a, kv_lens, off, U);
    const int32_t T = off[U];
    const int32_t per = (T + a.grid - 1) / a.grid;
    const int32_t c_begin = blockIdx.x * per;
    const int32_t c_end = min(c_begin + per, T);
    if (c_begin >= c_end) return;
    const int32_t total = c_end - c_begin;

    // unit holding c_begin: last u with off[u] <= c_begin
    int32_t lo_u = 0, hi_u = U - 1;
    while (lo_u < hi_u) {
        const int32_t mid = (lo_u + hi_u + 1) >> 1;
        if (off[mid] <= c_begin) lo_u = mid; else hi_u = mid - 1;
    }
    Unit ui = make_unit(a, kv_lens, lo_u);        // issue cursor
    int32_t ki = c_begin - off[lo_u];
    Unit uc = ui;                                 // compute cursor
    int32_t kc = ki;

    const int dq = wave * (D / 4);
    u32x4 qreg[C::KK];
    load_q<D>(a, uc, G, col, qg, dq, qreg);
    wait_vm<0>();   // Q has landed; nothing the compiler issued stays in flight under the copies
#pragma unroll
    for (int c = 0; c < C::NBUF - 1; ++c) {
        if (c < total) {
            issue_chunk<D, INT8>(a, page_table, lds + c * C::BUF, ui, ki, wave, lane);
            if (++ki == ui.n && ui.u + 1 < U) { ui = make_unit(a, kv_lens, ui.u + 1); ki = 0; }
        }
    }

    f32x4 o[C::MT];
    float m_run = -INFINITY, l_run = 0.0f;

    for (int32_t i = 0; i < total; ++i) {
        wait_chunks<C::PER, C::NBUF>(min(C::NBUF - 2, total - 1 - i));
        lds_barrier();
        if (kc == 0 || i == 0) {
            // a new unit inside the run: its Q (this load drains the copies in flight)
            if (i > 0) load_q<D>(a, uc, G, col, qg, dq, qreg);
#pragma unroll
            for (int m = 0; m < C::MT; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            l_run = 0.0f;
        }
        if (i + C::NBUF - 1 < total) {
            issue_chunk<D, INT8>(a, page_table, lds + ((i + C::NBUF - 1) % C::NBUF) * C::BUF, ui, ki, wave, lane);
            if (++ki == ui.n && ui.u + 1 < U) { ui = make_unit(a, kv_lens, ui.u + 1); ki = 0; }
        }
        const uint8_t* kbuf = lds + (i % C::NBUF) * C::BUF;
        const uint8_t* vbuf = kbuf + C::PAGE;
        const int32_t t0 = (uc.page0 + kc) * kChunk;

        // ---- partial scores over this wave's dim quarter --------------------
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const int row = col;
            const uint8_t* krow = kbuf + row * C::ROW;
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) {
                const int e0 = dq + 32 * kk + 8 * qg;          // first of 8 dims
                u32x4 ka;
                if constexpr (!INT8) {
                    ka = *reinterpret_cast<const u32x4*>(krow + (((e0 >> 3) ^ (row & 7)) * 16));
                } else {
                    const u32x2 w = *reinterpret_cast<const u32x2*>(krow + (((e0 >> 4) ^ (row & 7)) * 16) + (e0 & 8));
                    ka = u32x4{i8x2_to_bf16x2(w.x, 0), i8x2_to_bf16x2(w.x, 2),
                               i8x2_to_bf16x2(w.y, 0), i8x2_to_bf16x2(w.y, 2)};
                }
                acc = mfma_16x16x32(ka, qreg[kk], acc);
            }
        }
        sx[wave * 64 + lane] = acc;
        lds_barrier();
        f32x4 tot = sx[lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) tot += sx[w * 64 + lane];

        // ---- online softmax: lane holds tokens t0 + 4*qg + i -----------------
        float ks[4] = {1.f, 1.f, 1.f, 1.f}, vs[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (INT8) {
            const float* scl = reinterpret_cast<const float*>(vbuf + C::PAGE);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[e] = scl[4 * qg + e];
                vs[e] = scl[16 + 4 * qg + e];
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
            if constexpr (INT8) v *= ks[e];
            sc[e] = valid[e] ? v : -INFINITY;
            mx = fmaxf(mx, sc[e]);
        }
        mx = wave_max_across_groups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[4], psum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = exp2f(sc[e] - m_use);
            psum += p[e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = p[e];
            if constexpr (INT8) x *= vs[e];
            pv[e] = valid[e] ? x : 0.0f;
        }
        const u32x2 pb = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        const bool full = (t0 >= uc.lo) && (t0 + kChunk <= uc.hi);

        // ---- values: this wave's quarter of the output dims ------------------
#pragma unroll
        for (int m = 0; m < C::MT; ++m) {
            const int d = dq + 16 * m + col;
            u32x2 va;
            if constexpr (!INT8) {
                va = *reinterpret_cast<const u32x2*>(vbuf + d * 32 + 8 * qg);
                if (!full) {
                    va.x &= (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
                    va.y &= (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
                }
            } else {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(vbuf + d * 16 + 4 * qg);
                va = u32x2{i8x2_to_bf16x2(w, 0), i8x2_to_bf16x2(w, 2)};
            }
            o[m] = o[m] * alpha;
            o[m] = mfma_16x16x16(va, pb, o[m]);
        }

        // ---- end of this run's part of the unit --------------------------------
        if (kc == uc.n - 1 || i == total - 1) {
            const float l_tot = wave_sum_across_groups(l_run);
            const int32_t w0 = off[uc.u] / per, w1 = (off[uc.u + 1] - 1) / per;
            if (w0 == w1) {
                // the whole unit is in this run: normalise and write the outputs
                if (col < G) {
                    const float inv = 1.0f / l_tot;
                    uint16_t* op = a.out + ((int64_t)uc.b * a.hq + (int64_t)uc.g * G + col) * D + dq;
#pragma unroll
                    for (int m = 0; m < C::MT; ++m)
                        *reinterpret_cast<u32x2*>(op + 16 * m + 4 * qg) =
                            u32x2{pack_bf16x2(o[m][0] * inv, o[m][1] * inv), pack_bf16x2(o[m][2] * inv, o[m][3] * inv)};
                }
            } else {
                const int64_t slot = ((int64_t)blockIdx.x + uc.u) * G;
                if (col < G) {
                    float* po = a.part_o + (slot + col) * D + dq;
#pragma unroll
                    for (int m = 0; m < C::MT; ++m) put4(po + 16 * m + 4 * qg, o[m]);
                    if (wave == 0 && qg == 0) put2(a.part_ml + (slot + col) * 2, m_run, l_tot);
                }
                // the last of the unit's partials to arrive merges them all
                if (arrive_last(a.arrivals + uc.u, (uint32_t)(w1 - w0 + 1), &ticket)) {
                    merge_unit<D>(a, uc, w0, w1, G, threadIdx.x);
                    if (threadIdx.x == 0)
                        __hip_atomic_store(a.arrivals + uc.u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (++kc == uc.n && uc.u + 1 < U) { uc = make_unit(a, kv_lens, uc.u + 1); kc = 0; }
    }
    wait_vm<0>();
}

}  // namespace

namespace pakv {

int launch_decode(const DecodeLaunch& s, void* stream) {
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
    a.arrivals = s.arrivals;
    a.part_o = s.part_o;
    a.part_ml = s.part_ml;
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid1(s.plan.grid);
    const bool i8 = s.kv_dtype == PAKV_KV_INT8_PTH;
    const int K = PAKV_TIME_DECODE;
    if (s.head_dim == 256) {
        if (i8) launch(K, decode_kernel<256, true>, grid1, dim3(256), 0, st, a, s.page_table, s.kv_lens);
        else launch(K, decode_kernel<256, false>, grid1, dim3(256), 0, st, a, s.page_table, s.kv_lens);
    } else {
        if (i8) launch(K, decode_kernel<512, true>, grid1, dim3(256), 0, st, a, s.page_table, s.kv_lens);
        else launch(K, decode_kernel<512, false>, grid1, dim3(256), 0, st, a, s.page_table, s.kv_lens);
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
