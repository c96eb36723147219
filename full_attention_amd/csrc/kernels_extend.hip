// paged_attn_extend: chunked prefill over a paged cache with bf16 MFMA.
//
// One workgroup per (KV head g, sequence b, block of query rows).  Query rows
// are the (token, head) pairs of the G query heads that share KV head g,
// flattened token-major (row r = token * G + head), so each K/V tile staged in
// LDS serves every head of the group.  Each wavefront owns 32 rows and walks
// the workgroup's kv range in 32-token tiles (two pages), copied global -> LDS
// asynchronously one tile ahead:
//
//   S^T[32 kv x 32 rows] = K_tile . Q^T        D/16 MFMA 32x32x16
//   online softmax per row in the exp2 domain; the running max is raised (and
//   O rescaled) only when a tile's max passes it by more than 2^8, so the
//   accumulator is rarely touched by the VALU
//   O^T[D x 32 rows]    += V_tile^T . P^T      D/32 x 2 MFMA 32x32x16
//
// The score MFMA's row r = 8j + 4h + i reads kv token 16(j/2) + 8h + 4(j%2) + i,
// so the 16 scores a lane holds are kv tokens 8h..8h+7 and 16+8h..16+8h+7 of
// the tile: exactly the B operand the value MFMA wants in that lane, and P
// never goes through LDS.  V pages are dim-major, so the value MFMA's A operand
// (one dim, 8 consecutive tokens) is one 16-byte LDS read.
//
// D = 256: 8 wavefronts (256 rows) per workgroup, two per SIMD, Q^T and O^T in
// registers.  D = 512: 4 wavefronts (128 rows), one per SIMD, O^T in 256 AGPRs.
//
// Masks: the query row at position p sees kv position j iff j <= p and, on a
// sliding layer, p - j < W (unsloth commit ca9dbce, one block mask per regime;
// pegainfer issue #807, the window counts the query's own position).  Tiles
// visible to every row of a wavefront skip the mask arithmetic; elsewhere
// scores are selected to -inf.  Tokens of a tile outside the workgroup's kv
// range (slots never written, possibly NaN) have their V zeroed in LDS so that
// P = 0 times V stays 0.

#include "async_copy.h"
#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;            // kv tokens per staged tile (two pages)
constexpr float kRescale = 8.0f;     // raise the running max only past 2^8

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// The D = 512 kernel keeps O^T in all 256 AGPRs; a compiler-selected score
// MFMA would also take its accumulator from the AGPR file and force spills, so
// the score chain is issued as VGPR-form MFMAs in inline assembly.  The
// compiler's hazard tracking does not see inside the asm: each MFMA is preceded
// by s_nop 2 (VALU write -> MFMA read of a source), consecutive MFMAs share the
// accumulator exactly (back-to-back accumulation needs no wait states), and the
// chain ends with 24 wait states before any VALU may read or overwrite it.
__device__ __forceinline__ f32x16 asm_mfma_first(u32x4 a, u32x4 b) {
    f32x16 c;
    asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    return c;
}
__device__ __forceinline__ void asm_mfma_acc(f32x16& c, u32x4 a, u32x4 b) {
    asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void asm_mfma_drain(f32x16& c) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

// o *= al for an accumulator tile that lives in AGPRs, written as explicit
// AGPR read / multiply / write so that the compiler keeps the tile in the AGPR
// file across the loop.  Called at most a few times per workgroup; it is
// fenced by wait states for the MFMA that last wrote the tile and for the
// MFMA that next reads it.
__device__ __forceinline__ void agpr_scale(f32x16& o, float al) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float x = o[e], t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(t)
            : "v"(al));
        o[e] = x;
    }
    asm volatile("s_nop 4" ::: "memory");
}

// Pins a tile to the AGPR file at this point (no instruction is emitted), so
// the loop-carried accumulators are not copied into VGPRs at the back edge.
__device__ __forceinline__ void pin_agpr(f32x16& o) { asm volatile("" : "+a"(o)); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

// Exchange between the two halves of the wave: v_permlane32_swap swaps lanes
// 32..63 of its first operand with lanes 0..31 of its second, so with x in
// both, lane l ends up holding x[l % 32] in `lo` and x[l % 32 + 32] in `hi`.
// (Written as asm: the compiler builtin folded the two results into one.)
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
    lo = x;
    hi = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ float max_halves(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return lo + hi;
}

struct ExtendArgs {
    const uint16_t* k_slab;
    const uint16_t* v_slab;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_q;
    const int32_t* prefix_lens;
    const uint16_t* q;
    uint16_t* out;
    int32_t max_q_len;
    int32_t max_kv_len;
    int32_t hq;
    int32_t hkv;
    int32_t group;
    int32_t window;
    float score_scale;   // sm_scale * log2(e)
};

// XOR key of a kv token's K row in LDS (16-byte granules): the 8 rows that 8
// consecutive lanes read land in 8 different bank groups.
__device__ __forceinline__ int k_swz(int tk) { return (tk & 3) | ((tk >> 1) & 4); }

template <int D>
struct XCfg {
    static constexpr int NW = (D == 256) ? 8 : 4;       // wavefronts per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int ROWS = 32 * NW;                // query rows per workgroup
    static constexpr int KROW = D * 2;                  // bytes per K row
    static constexpr int PAGE = 16 * D * 2;             // bytes per (page, head) block
    static constexpr int TILE = 4 * PAGE;               // K (2 pages) + V (2 pages)
    static constexpr int NBUF = 2;
    static constexpr int DMA = TILE / 1024 / NW;         // 1 KiB copies per wave per tile
    static constexpr int LDS = NBUF * TILE;
    static constexpr int KK = D / 16;                   // 16-dim steps of the score product
    static constexpr int MT = D / 32;                   // 32-dim tiles of the output
    static_assert(DMA % 2 == 0 && DMA * NW * 1024 == TILE, "tile copies must split evenly");
};

// Copies K and V of the tile whose two pages are physical pages ph0, ph1.
// Copy `inst` of the K region fills LDS bytes [1024 inst, +1024): K rows
// tk = inst * 64 / (D / 8) + lane / (D / 8), with granule colp ^ key(tk) of
// row tk landing at granule colp.  Copy `inst` of the V region fills dims
// d = 32 inst + lane / 2 (page inst / (D / 32)), half (lane & 1) ^ bit 2 of d.
template <int D>
__device__ __forceinline__ void issue_tile(const ExtendArgs& a, uint32_t kb, int32_t ph0, int32_t ph1, int32_t g,
                                           int wave, int lane) {
    using C = XCfg<D>;
    constexpr int GR = C::KROW / 16;                    // granules per K row (32 or 64)
    const uint32_t vb = kb + 2 * C::PAGE;
    const uint8_t* kbase[2] = {
        reinterpret_cast<const uint8_t*>(a.k_slab) + ((int64_t)ph0 * a.hkv + g) * C::PAGE,
        reinterpret_cast<const uint8_t*>(a.k_slab) + ((int64_t)ph1 * a.hkv + g) * C::PAGE};
    const uint8_t* vbase[2] = {
        reinterpret_cast<const uint8_t*>(a.v_slab) + ((int64_t)ph0 * a.hkv + g) * C::PAGE,
        reinterpret_cast<const uint8_t*>(a.v_slab) + ((int64_t)ph1 * a.hkv + g) * C::PAGE};
    const int colp = lane % GR;
    const int v_lane = (lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 3) & 1)) * 16);
#pragma unroll
    for (int i = 0; i < C::DMA / 2; ++i) {
        const int inst = wave + C::NW * i;                      // wave-uniform
        const int tk = (inst * 64 + lane) / GR;                 // uniform when GR = 64
        const uint32_t off = (tk & 15) * C::KROW + ((colp ^ k_swz(tk)) * 16);
        dma16_s(kbase[(inst * 64) / (16 * GR)], off, kb + inst * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::DMA / 2; ++i) {
        const int inst = wave + C::NW * i;
        const int p = inst / (D / 32);
        const uint32_t off = (inst % (D / 32)) * 1024 + v_lane;
        dma16_s(vbase[p], off, vb + inst * 1024);
    }
}

template <int D>
__global__ __launch_bounds__(XCfg<D>::THREADS) void extend_kernel(ExtendArgs a) {
    using C = XCfg<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    // grid (Hkv, B, row blocks): dispatch walks x fastest, so every (head,
    // sequence) pair gets its heaviest (last) row block before any lighter one
    const int32_t g = blockIdx.x, b = blockIdx.y;
    const int32_t blk = gridDim.z - 1 - blockIdx.z;
    const int32_t G = a.group;
    const int32_t q0 = a.cu_q[b];
    const int32_t n = min(a.cu_q[b + 1] - q0, a.max_q_len);
    const int32_t prefix = a.prefix_lens[b];
    const int32_t rows = n * G;
    const int32_t row0 = blk * C::ROWS;
    if (n <= 0 || row0 >= rows) return;

    const int32_t tok_first = row0 / G;
    const int32_t tok_last = min(n - 1, (row0 + C::ROWS - 1) / G);
    const int32_t hi = min(prefix + tok_last + 1, a.max_kv_len);          // kv range of the workgroup
    const int32_t lo = (a.window > 0) ? max(0, prefix + tok_first - a.window + 1) : 0;

    // this lane's query row (score column) and its visible kv range [row_lo, row_hi]
    const int32_t wrow0 = row0 + wave * 32;
    const bool wave_live = wrow0 < rows;
    const int32_t my_row = wrow0 + col;
    const bool row_ok = my_row < rows;
    const int32_t my_tok = row_ok ? my_row / G : 0, my_head = my_row % G;
    const int32_t my_pos = prefix + my_tok;
    const int32_t row_hi = min(my_pos, hi - 1);
    const int32_t row_lo = (a.window > 0) ? my_pos - a.window + 1 : -(1 << 30);
    // the wavefront's extreme positions, for the "tile visible to all rows" test
    const int32_t w_pmin = prefix + min(n - 1, wrow0 / G);
    const int32_t w_pmax = prefix + min(n - 1, (wrow0 + 31) / G);

    const int32_t t_begin = (lo / kTile) * kTile;
    const int32_t n_tiles = (hi - t_begin + kTile - 1) / kTile;
    const int32_t page0 = t_begin / 16;

    // page ids of pages page0 + 64c + lane, batch c; missing pages read page 0
    const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
    auto load_ids = [&](int32_t c) -> int32_t {
        const int32_t pg = page0 + 64 * c + lane;
        int32_t ph = 0;
        if (pg < a.max_pages) ph = pt[pg];
        return ((uint32_t)ph < (uint32_t)a.num_pages) ? ph : 0;
    };
    int32_t ids = load_ids(0);
    int32_t ids_next = (n_tiles > 32) ? load_ids(1) : 0;

    // Q^T operand: lane holds Q[row col][16 kk + 8 h .. +8]; rows past the
    // chunk read token 0 of the chunk and are never written back
    u32x4 qreg[C::KK];
    {
        const uint16_t* qp = a.q + ((int64_t)(q0 + my_tok) * a.hq + (int64_t)g * G + my_head) * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4*>(qp + 16 * kk);
    }
    wait_vm<0>();

    const uint32_t lds0 = lds_addr_of(lds);
    if (n_tiles > 0)
        issue_tile<D>(a, lds0, __builtin_amdgcn_readlane(ids, 0), __builtin_amdgcn_readlane(ids, 1), g, wave, lane);

    f32x16 o[C::MT];
#pragma unroll
    for (int m = 0; m < C::MT; ++m) o[m] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    if constexpr (D == 512) {
#pragma unroll
        for (int m = 0; m < C::MT; ++m) pin_agpr(o[m]);
    }

    // LDS offsets this lane reads: K row tau(col), granules (2 kk + h) ^ key
    int k_off[4];
    {
        const int j = col >> 3, hh = (col >> 2) & 1, i = col & 3;
        const int tk = 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
#pragma unroll
        for (int s = 0; s < 4; ++s) k_off[s] = tk * C::KROW + (((2 * s + h) ^ k_swz(tk)) * 16);
    }
    const int v_off = col * 32 + ((h ^ ((col >> 2) & 1)) * 16);

    for (int32_t it = 0; it < n_tiles; ++it) {
        wait_vm<0>();
        lds_barrier();
        const int32_t t0 = t_begin + it * kTile;
        if (it + 1 < n_tiles) {
            const int32_t rp = 2 * (it + 1);            // page of the next tile, relative to page0
            if ((rp & 63) == 0) {
                ids = ids_next;
                if (it + 33 < n_tiles) ids_next = load_ids((rp >> 6) + 1);
            }
            issue_tile<D>(a, lds0 + ((it + 1) % C::NBUF) * C::TILE, __builtin_amdgcn_readlane(ids, rp & 63),
                          __builtin_amdgcn_readlane(ids, (rp & 63) + 1), g, wave, lane);
        }
        uint8_t* kbuf = lds + (it % C::NBUF) * C::TILE;
        uint8_t* vbuf = kbuf + 2 * C::PAGE;
        if (t0 < lo || t0 + kTile > hi) {
            // zero V of tokens outside [lo, hi): never-written slots may hold NaN
            for (int idx = tid; idx < 4 * D; idx += C::THREADS) {
                const int p = idx / (2 * D), d = (idx >> 1) % D, hp = idx & 1;
                const int half = hp ^ ((d >> 2) & 1);
                const int32_t tb = t0 + 16 * p + 8 * half;
                u32x4* gp = reinterpret_cast<u32x4*>(vbuf + p * C::PAGE + d * 32 + hp * 16);
                u32x4 v = *gp;
                uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t t = tb + 2 * e;
                    const uint32_t keep = ((t >= lo && t < hi) ? 0xffffu : 0u) |
                                          ((t + 1 >= lo && t + 1 < hi) ? 0xffff0000u : 0u);
                    w[e] &= keep;
                }
                *gp = u32x4{w[0], w[1], w[2], w[3]};
            }
            lds_barrier();
        }
        if (wave_live) {
        // ---- scores S^T[kv][row col] -------------------------------------------------
        f32x16 s;
        if constexpr (D == 512) {
            s = asm_mfma_first(*reinterpret_cast<const u32x4*>(kbuf + k_off[0]), qreg[0]);
#pragma unroll
            for (int kk = 1; kk < C::KK; ++kk)
                asm_mfma_acc(s, *reinterpret_cast<const u32x4*>(kbuf + k_off[kk & 3] + (kk >> 2) * 128), qreg[kk]);
            asm_mfma_drain(s);
        } else {
            s = f32x16{};
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(kbuf + k_off[kk & 3] + (kk >> 2) * 128);
                s = mfma_32x32x16(ka, qreg[kk], s);
            }
        }
        const bool whole = (t0 + kTile - 1 <= min(w_pmin, hi - 1)) &&
                           (a.window == 0 || w_pmax - a.window + 1 <= t0);
        if (!whole) {
            // element e holds kv offset 8h + e + 8 (e >= 8) of the tile
            const int32_t lo_l = row_lo - t0 - 8 * h, hi_l = row_hi - t0 - 8 * h;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = e + ((e >> 3) << 3);
                s[e] = ((c >= lo_l) & (c <= hi_l)) ? s[e] : -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = max_halves(mx) * a.score_scale;
        const bool raise = mx > m_run + kRescale;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float m_new = raise ? mx : m_run;
            const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float al = raise ? alpha : 1.f;
            l_run *= al;
            m_run = m_new;
            if constexpr (D == 512) {
#pragma unroll
                for (int m = 0; m < C::MT; ++m) agpr_scale(o[m], al);
            } else {
#pragma unroll
                for (int m = 0; m < C::MT; ++m) o[m] *= al;
            }
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.score_scale, -m_use));
            l_run += s[e];
        }
        u32x4 pb[2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
            pb[st] = u32x4{cvt_pk_bf16(s[8 * st + 0], s[8 * st + 1]), cvt_pk_bf16(s[8 * st + 2], s[8 * st + 3]),
                           cvt_pk_bf16(s[8 * st + 4], s[8 * st + 5]), cvt_pk_bf16(s[8 * st + 6], s[8 * st + 7])};

        // ---- values O^T[d][row] += V^T[d][kv] P^T[kv][row] ---------------------------
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int m = 0; m < C::MT; ++m) {
                const u32x4 va = *reinterpret_cast<const u32x4*>(vbuf + st * C::PAGE + m * 1024 + v_off);
                o[m] = mfma_32x32x16(va, pb[st], o[m]);
            }
        }
        }
        if constexpr (D == 512) {
#pragma unroll
            for (int m = 0; m < C::MT; ++m) pin_agpr(o[m]);
        }
    }

    wait_vm<0>();   // no copy may still be landing in LDS when the workgroup ends
    l_run = sum_halves(l_run);
    if (!row_ok) return;
    const float inv = 1.0f / l_run;
    uint16_t* op = a.out + ((int64_t)(q0 + my_tok) * a.hq + (int64_t)g * G + my_head) * D;
#pragma unroll
    for (int m = 0; m < C::MT; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 32 * m + 8 * j + 4 * h;
            *reinterpret_cast<u32x2*>(op + d) = u32x2{cvt_pk_bf16(o[m][4 * j] * inv, o[m][4 * j + 1] * inv),
                                                      cvt_pk_bf16(o[m][4 * j + 2] * inv, o[m][4 * j + 3] * inv)};
        }
    }
}

}  // namespace

namespace pakv {

int launch_extend(const ExtendLaunch& s, void* stream) {
    ExtendArgs a;
    a.k_slab = static_cast<const uint16_t*>(s.slab.k);
    a.v_slab = static_cast<const uint16_t*>(s.slab.v);
    a.num_pages = s.slab.num_pages;
    a.page_table = s.page_table;
    a.max_pages = s.max_pages;
    a.cu_q = s.cu_q;
    a.prefix_lens = s.prefix_lens;
    a.q = s.q;
    a.out = s.out;
    a.max_q_len = s.max_q_len;
    a.max_kv_len = s.max_kv_len;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.group = s.hq / s.hkv;
    a.window = s.window;
    a.score_scale = s.sm_scale * kLog2e;
    const int64_t rows = (int64_t)s.max_q_len * a.group;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.head_dim == 256) {
        using C = XCfg<256>;
        const dim3 grid(s.hkv, s.num_seqs, (unsigned)((rows + C::ROWS - 1) / C::ROWS));
        launch(PAKV_TIME_EXTEND, extend_kernel<256>, grid, dim3(C::THREADS), 0, st, a);
    } else {
        using C = XCfg<512>;
        const dim3 grid(s.hkv, s.num_seqs, (unsigned)((rows + C::ROWS - 1) / C::ROWS));
        launch(PAKV_TIME_EXTEND, extend_kernel<512>, grid, dim3(C::THREADS), 0, st, a);
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
