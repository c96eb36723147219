// paged_attn_extend: chunked prefill over a paged cache with bf16 MFMA.
//
// One workgroup per (KV head g, sequence b, block of query rows).  Query rows
// are the (token, head) pairs of the G query heads that share KV head g,
// flattened token-major (row r = token * G + head), so each K/V tile staged in
// LDS serves every head of the group.  Each wavefront owns 32 rows and walks
// the workgroup's kv range in 32-token tiles (two pages), copied global -> LDS
// asynchronously ahead of use:
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
// Four wavefronts per workgroup, each owning 32 rows (128 rows per
// workgroup); O^T lives in AGPRs (D/32 tiles), Q^T and the score tiles in
// VGPRs.  At D = 512 a workgroup has its CU (one wavefront per SIMD); at
// D = 256 two workgroups share a CU.  K and V have rings of
// two tiles each, and a wavefront's step t runs the score product of tile t+1
// and the value product of tile t interleaved (two independent MFMA chains),
// then the softmax of tile t+1; K(t+2) and V(t+1) are copied meanwhile.
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
constexpr int kRankedSeqs = 256;     // sequences ordered by weight at dispatch (one per thread)
constexpr float kRescale = 8.0f;     // raise the running max only past 2^8
constexpr int kRuns = 4;             // copy runs per step: V(t+1) and K(t+2), one per page

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
// Value MFMA with its accumulator tile held in AGPRs (the "a" constraint keeps
// the tile there).  Its B operand (P^T) is written by the VALU shortly before
// the first value MFMA of a step, which therefore takes the s_nop form.
__device__ __forceinline__ void asm_mfma_agpr(f32x16& c, u32x4 a, u32x4 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void asm_mfma_agpr_nop(f32x16& c, u32x4 a, u32x4 b) {
    asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// o *= al for an accumulator tile that lives in AGPRs, written as explicit
// AGPR read / multiply / write so that the compiler keeps the tile in the AGPR
// file across the loop.  Called at most a few times per workgroup, after
// settle_tiles() (the MFMAs that last wrote the tiles have landed); it ends
// with the wait states the next MFMA that reads the tile needs.
__device__ __forceinline__ void agpr_scale(f32x16& o, float al) {
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

// 24 wait states that every accumulator tile passes through: the value MFMAs
// are inline asm, so the compiler does not know that the tiles are written by
// an MFMA still in flight, and any read it schedules (a copy, a rescale, the
// output) must come after this statement, which takes all tiles as operands.
#define PAKV_SETTLE "s_nop 7\n\ts_nop 7\n\ts_nop 7"
__device__ __forceinline__ void settle_tiles(f32x16 (&o)[8]) {
    asm volatile(PAKV_SETTLE : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                 "+a"(o[7]));
}
__device__ __forceinline__ void settle_tiles(f32x16 (&o)[16]) {
    asm volatile(PAKV_SETTLE : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                 "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));
}
#undef PAKV_SETTLE

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
    float inv_group;     // 1 / group, as a float
    uint32_t* bad_ids;   // counters of a PAKV_DEBUG_BOUNDS build, else null
    // staged call (the scaled kernel): the slab is the staging workspace of
    // kernels_extend_stage.hip -- sequence b's pages from the tile of its
    // first row's start at b * stage_stride, stage_pages in all -- and
    // stage_scales holds per (KV head, page) the 16 key scales then the 16
    // value scales of its tokens, [Hkv][stage_pages][32] floats
    const float* stage_scales;
    int32_t stage_stride;
    int32_t stage_pages;
};

// XOR key of a kv token's K row in LDS (16-byte granules).  LDS serves a
// 16-byte-per-lane read 16 lanes at a time over 64 banks; the 16 rows that 16
// consecutive lanes read land in 16 different bank groups.
__device__ __forceinline__ int k_swz(int tk) { return tk & 15; }

// LDS byte offsets, within a K tile slot, of the 16 bytes a lane reads at
// score step kk: granule 2 kk + h of its K row tk, XOR the row's key.  With
// base = tk * row bytes + ((h ^ key) * 16), granule 16 c + 8 a + 2 b + h
// (kk = 8 c + 4 a + b) lies at base ^ ((8 a + 2 b) * 16), plus 256 c: the
// key and 8 a + 2 b + h only touch bits 4..7, and h is their bit 4.  At
// D = 256 (two wavefronts per SIMD, registers short) the offset is formed at
// each read from the base; at D = 512 (one wavefront per SIMD, whose own
// VALU work is not hidden) the 8 XORed offsets are kept.
template <int D>
struct KOffsets {
    static constexpr int N = (D == 256) ? 1 : 8;
    int v[N];
    __device__ __forceinline__ void init(int base) {
        if constexpr (N == 1) v[0] = base;
        else
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) v[s8] = base ^ ((8 * (s8 >> 2) + 2 * (s8 & 3)) * 16);
    }
    __device__ __forceinline__ int operator()(int kk) const {
        if constexpr (N == 1) return (v[0] ^ ((8 * ((kk >> 2) & 1) + 2 * (kk & 3)) * 16)) + (kk >> 3) * 256;
        else return v[((kk >> 2) & 1) * 4 + (kk & 3)] + (kk >> 3) * 256;
    }
};

template <int D>
struct XCfg {
    static constexpr int NW = 4;                        // wavefronts per workgroup, one per SIMD
    static constexpr int THREADS = 64 * NW;
    // one 32-row block per wavefront.  At D = 512 its O^T fills the 256
    // AGPRs and the workgroup has the CU; at D = 256 a wavefront fits in 256
    // registers, so two workgroups share a CU and one's softmax, prologue and
    // output overlap the other's matrix work (with two blocks per wavefront
    // and one workgroup per CU the sliding launch was ~8% slower)
    static constexpr int NRB = 1;
    static constexpr int OT = NRB * (D / 32);           // accumulator tiles of O^T
    static constexpr int MINB = (D == 256) ? 2 : 1;     // workgroups per CU
    // LDS operands prefetched ahead of the MFMAs; at D = 256 deeper
    // prefetch spills
    static constexpr int PF = (D == 256) ? 2 : 4;
    static constexpr int ROWS = 32 * NRB * NW;          // query rows per workgroup
    static constexpr int KROW = D * 2;                  // bytes per K row
    static constexpr int PAGE = 16 * D * 2;             // bytes per (page, head) block
    static constexpr int HALF = 2 * PAGE;               // K (or V) of one 32-token tile
    static constexpr int PP = PAGE / 1024;              // 1 KiB pieces per (page, head) block
    static constexpr int NI = PP / NW;                  // pieces per wavefront per page
    static constexpr int LDS = (4 * HALF > ROWS * D * 2) ? 4 * HALF : ROWS * D * 2;   // K, V rings; the output rows
    static constexpr int KK = D / 16;                   // 16-dim steps of the score product
    static constexpr int MT = D / 32;                   // 32-dim tiles of the output
    static_assert(KK == 2 * MT, "one score MFMA per value MFMA");
    static_assert(NI * NW == PP && (NI == 2 || NI == 4), "page copies must split into runs of 2 or 4");
};

// Each (page, head) block of K or V is PP = PAGE / 1 KiB pieces; wavefront w
// copies pieces NI w .. NI w + NI - 1 (NI = PP / NW) of every page of a tile,
// piece q of page p landing at LDS bytes [1024 (PP p + q), +1024), as one run
// of NI copies with M0 written once (copy i of a run carries the immediate
// offset 1024 i, added to both addresses).
//
// K piece q holds the page's rows tk = (64 q + lane) / GR (GR 16-byte
// granules per row), granule colp ^ key(tk) of row tk landing at granule colp;
// V piece q holds dims d = 32 q + lane / 2 of the page, half (lane & 1) ^
// bit 3 of d.  The per-lane source offsets (less 1024 i) are the same for
// every page and every tile, so they are formed once.
template <int D>
__device__ __forceinline__ void copy_offsets(int wave, int lane, uint32_t (&k_voff)[XCfg<D>::NI], uint32_t& v_voff) {
    using C = XCfg<D>;
    constexpr int GR = C::KROW / 16;
    const int colp = lane % GR;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
        const int q = C::NI * wave + i;
        const int tk = (q * 64 + lane) / GR;
        k_voff[i] = (uint32_t)(tk * C::KROW + ((colp ^ k_swz(tk)) * 16) - 1024 * i);
    }
    v_voff = (uint32_t)(C::NI * wave * 1024 + (lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 4) & 1)) * 16));
}

// One wavefront's run of page p of a tile (LDS slot base `slot`) from the
// block at `src` (K: per-piece offsets k_voff; V: v_voff for every piece).
template <int D>
__device__ __forceinline__ void copy_k_run(const uint8_t* src, const uint32_t (&k_voff)[XCfg<D>::NI], uint32_t slot,
                                           int p, int wave) {
    using C = XCfg<D>;
    const uint32_t dst = slot + (C::PP * p + C::NI * wave) * 1024;
    if constexpr (C::NI == 4) dma16_s_x4(src, k_voff[0], k_voff[1], k_voff[2], k_voff[3], dst);
    else dma16_s_x2(src, k_voff[0], k_voff[1], dst);
}
// Copy i alone of the K (or V) run of page p.
template <int D, int I>
__device__ __forceinline__ void copy_k_one(const uint8_t* src, const uint32_t (&k_voff)[XCfg<D>::NI], uint32_t slot,
                                           int p, int wave) {
    using C = XCfg<D>;
    dma16_s_at<I>(src, k_voff[I], slot + (C::PP * p + C::NI * wave) * 1024);
}
template <int D, int I>
__device__ __forceinline__ void copy_v_one(const uint8_t* src, uint32_t v_voff, uint32_t slot, int p, int wave) {
    using C = XCfg<D>;
    dma16_s_at<I>(src, v_voff, slot + (C::PP * p + C::NI * wave) * 1024);
}
template <int D>
__device__ __forceinline__ void copy_v_run(const uint8_t* src, uint32_t v_voff, uint32_t slot, int p, int wave) {
    using C = XCfg<D>;
    const uint32_t dst = slot + (C::PP * p + C::NI * wave) * 1024;
    if constexpr (C::NI == 4) dma16_s_x4(src, v_voff, v_voff, v_voff, v_voff, dst);
    else dma16_s_x2(src, v_voff, v_voff, dst);
}

// Copy i of the run of page p: K (is_k) or V, i known once the loops unroll.
template <int D>
__device__ __forceinline__ void copy_piece(bool is_k, int i, const uint8_t* src, const uint32_t (&k_voff)[XCfg<D>::NI],
                                           uint32_t v_voff, uint32_t slot, int p, int wave) {
    if (is_k) {
        if (i == 0) copy_k_one<D, 0>(src, k_voff, slot, p, wave);
        else if (i == 1) copy_k_one<D, 1>(src, k_voff, slot, p, wave);
        if constexpr (XCfg<D>::NI == 4) {
            if (i == 2) copy_k_one<D, 2>(src, k_voff, slot, p, wave);
            else if (i == 3) copy_k_one<D, 3>(src, k_voff, slot, p, wave);
        }
    } else {
        if (i == 0) copy_v_one<D, 0>(src, v_voff, slot, p, wave);
        else if (i == 1) copy_v_one<D, 1>(src, v_voff, slot, p, wave);
        if constexpr (XCfg<D>::NI == 4) {
            if (i == 2) copy_v_one<D, 2>(src, v_voff, slot, p, wave);
            else if (i == 3) copy_v_one<D, 3>(src, v_voff, slot, p, wave);
        }
    }
}

// Online softmax of one score tile, in stages that the step spreads over its
// value MFMAs (lane: query row col; s holds the row's scores of kv tokens
// 8h..8h+7 and 16+8h..16+8h+7 of the tile at t0).  Stage 0 masks the tile
// where it is not visible to every row and takes the max of the first eight
// scores; stage 1 finishes the max and updates the running max, raised only
// when the tile's max passes it by more than 2^8 (the factor `al` for O and
// the wave-wide flag `raise` are left for the caller, which scales O before
// the next value product); stages 2-5 exponentiate four scores each into s
// and add them to the row sum; stage 6 packs the first kv half into pb0.  The
// second half is packed by softmax_pack_hi once the value MFMAs of the
// current tile no longer read pb1.
// The lane id, recomputed where it is used (the asm keeps the compiler from
// holding it, or a value derived from it, across the main loop: the D = 256
// kernel has no register to spare for them and spilled them to scratch).
__device__ __forceinline__ int32_t lane_id_here() {
    int32_t v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

struct SoftRow {
    float mx;
    float m_use;
    float al;
    bool raise;
};

// The row's visible kv range is [row_lo, row_hi].  FRESH (the D = 256
// kernel): the row's position, the range (lower end position - window + 1 on
// a sliding layer, upper min(position, hi - 1), given as row_hi) and the
// lane's 8h are formed here, out of values the compiler cannot hoist: kept
// across the loop they took registers it does not have.  The position is
// row_lo + floor((row_r + col) / G) for the lane's column col, with the
// wave-uniform row_lo (prefix + first row / G), row_r (first row mod G) and
// inv_g = 1 / G: (x + 1/2) / G lies at least 1/(2G) from an integer, far
// beyond the float product's error, so the floor is exact.
// SC (the staged kernel): sc holds the tile's scales, per page the 16 key
// scales then the 16 value scales of its tokens; stage 0 multiplies each
// score by its key's scale before anything else, and the packing multiplies
// each weight by its key's value scale (the row sum takes the weights as
// they are).
template <bool FRESH, bool SC>
__device__ __forceinline__ void softmax_stage(int stage, f32x16& s, SoftRow& r, int32_t t0, bool whole,
                                              int32_t row_lo, int32_t row_hi, int32_t window, int h,
                                              float score_scale, float& m_run, float& l_run, u32x4& pb0,
                                              const float* sc, int32_t row_r, float inv_g) {
    if (stage == 0) {
        if constexpr (SC) {
            const int h8 = (lane_id_here() >> 5) << 3;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {           // tokens h8 .. h8 + 7, then 16 + h8 .. + 7
                const f32x4 k0 = *reinterpret_cast<const f32x4*>(sc + 32 * hf + h8);
                const f32x4 k1 = *reinterpret_cast<const f32x4*>(sc + 32 * hf + h8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s[8 * hf + e] *= k0[e];
                    s[8 * hf + 4 + e] *= k1[e];
                }
            }
        }
        if (!whole) {
            // element e holds kv offset 8h + e + 8 (e >= 8) of the tile
            int32_t lo_l, hi_l;
            if constexpr (FRESH) {
                const int32_t lid = lane_id_here();
                const int32_t h8 = (lid >> 5) << 3;
                const int32_t pos = row_lo + (int32_t)(((float)(row_r + (lid & 31)) + 0.5f) * inv_g);
                lo_l = (window > 0 ? pos - window + 1 : -(1 << 30)) - t0 - h8;
                hi_l = min(pos, row_hi) - t0 - h8;
            } else {
                lo_l = row_lo - t0 - 8 * h;
                hi_l = row_hi - t0 - 8 * h;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = e + ((e >> 3) << 3);
                s[e] = ((c >= lo_l) & (c <= hi_l)) ? s[e] : -INFINITY;
            }
        }
        r.mx = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) r.mx = fmaxf(r.mx, s[e]);
    } else if (stage == 1) {
        float mx = r.mx;
#pragma unroll
        for (int e = 8; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = max_halves(mx) * score_scale;
        const bool raise = mx > m_run + kRescale;
        r.raise = __builtin_amdgcn_ballot_w64(raise) != 0;
        const float m_new = raise ? mx : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        r.al = raise ? alpha : 1.f;
        l_run *= r.al;
        m_run = m_new;
        r.m_use = (m_run == -INFINITY) ? 0.f : m_run;
    } else if (stage <= 5) {
        const int e0 = 4 * (stage - 2);
#pragma unroll
        for (int e = e0; e < e0 + 4; ++e) {
            s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], score_scale, -r.m_use));
            l_run += s[e];
        }
    } else if (stage == 6) {
        if constexpr (SC) {
            const int h8 = (lane_id_here() >> 5) << 3;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(sc + 16 + h8);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(sc + 16 + h8 + 4);
            // (every staged scale is finite, zero outside the staged range,
            // so a masked key's weight 0 stays 0)
            pb0 = u32x4{cvt_pk_bf16(s[0] * v0[0], s[1] * v0[1]), cvt_pk_bf16(s[2] * v0[2], s[3] * v0[3]),
                        cvt_pk_bf16(s[4] * v1[0], s[5] * v1[1]), cvt_pk_bf16(s[6] * v1[2], s[7] * v1[3])};
        } else {
            pb0 = u32x4{cvt_pk_bf16(s[0], s[1]), cvt_pk_bf16(s[2], s[3]), cvt_pk_bf16(s[4], s[5]),
                        cvt_pk_bf16(s[6], s[7])};
        }
    }
}
constexpr int kSoftStages = 7;
template <bool SC>
__device__ __forceinline__ void softmax_pack_hi(const f32x16& s, u32x4& pb1, const float* sc) {
    if constexpr (SC) {
        const int h8 = (lane_id_here() >> 5) << 3;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(sc + 48 + h8);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(sc + 48 + h8 + 4);
        pb1 = u32x4{cvt_pk_bf16(s[8] * v0[0], s[9] * v0[1]), cvt_pk_bf16(s[10] * v0[2], s[11] * v0[3]),
                    cvt_pk_bf16(s[12] * v1[0], s[13] * v1[1]), cvt_pk_bf16(s[14] * v1[2], s[15] * v1[3])};
    } else {
        pb1 = u32x4{cvt_pk_bf16(s[8], s[9]), cvt_pk_bf16(s[10], s[11]), cvt_pk_bf16(s[12], s[13]),
                    cvt_pk_bf16(s[14], s[15])};
    }
}

// One wavefront's step of the software pipeline: the score product of tile
// t+1 (kb) runs first, a chain of D/16 MFMAs per row block at full rate, then
// the value product of tile t (vb, operands pb), D/16 MFMAs per row block,
// with soft(i) between them: the stages of the softmax of tile t+1, whose
// scores are complete by then; soft_end() packs what the value MFMAs read
// last.  Each K or V operand read from LDS feeds the MFMAs of all NRB row
// blocks of the wavefront.  The LDS operands are prefetched a few MFMAs
// ahead in rotating registers, and a scheduling barrier closes every loop
// step so the compiler keeps this order (and this register footprint)
// instead of hoisting every load.  copy(c) issues copy c (of at most
// kRuns * NI) of the next tiles' global -> LDS copies.  The copies are spread
// one every few loop steps over both loops: a copy holds up the wavefront
// that issues it while the CU's address unit works through the copies ahead
// of it, so issued together they stall the matrix work.  With HAVE_S = false
// only the value product runs (the last tile).
template <int D, bool HAVE_S, typename Copy, typename Soft, typename SoftEnd>
__device__ __forceinline__ void step_mfma(const uint8_t* kb, const uint8_t* vb, const KOffsets<D>& k_off, int v_off,
                                          const u32x4 (&qreg)[XCfg<D>::NRB][D / 16],
                                          const u32x4 (&pb)[XCfg<D>::NRB][2], f32x16 (&s)[XCfg<D>::NRB],
                                          f32x16 (&o)[XCfg<D>::OT], int n_copies, Copy copy, Soft soft, SoftEnd soft_end) {
    constexpr int KK = D / 16, MT = D / 32, PFK = XCfg<D>::PF, PFV = XCfg<D>::PF, NRB = XCfg<D>::NRB;
    constexpr int kCopies = kRuns * XCfg<D>::NI;                  // copies per wavefront per step
    constexpr int kCopyGap = (2 * KK) / kCopies;                   // loop steps between copies
    static_assert(kCopyGap >= 1 && (kCopies - 1) * kCopyGap < 2 * KK, "every copy needs a loop step");
    // loop step e of the step (score loop e = j, value loop e = KK + i)
    auto copy_at = [&](int e) {
        if (e % kCopyGap == 0 && e / kCopyGap < kCopies) {
            if (e / kCopyGap < n_copies) copy(e / kCopyGap);
        }
    };
    // score step i: granules 2i + h of the lane's K row
    auto ld_k = [&](int i) { return *reinterpret_cast<const u32x4*>(kb + k_off(i)); };
    // value step i: kv half st = i / MT, output tile m = i % MT
    auto ld_v = [&](int i) {
        return *reinterpret_cast<const u32x4*>(vb + (i / MT) * (16 * D * 2) + (i % MT) * 1024 + v_off);
    };
    u32x4 kr[PFK], vr[PFV];
    if constexpr (HAVE_S) {
#pragma unroll
        for (int p = 0; p < PFK; ++p) kr[p] = ld_k(p);
#pragma unroll
        for (int j = 0; j < KK; ++j) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                if (j == 0) s[rb] = asm_mfma_first(kr[0], qreg[rb][0]);
                else asm_mfma_acc(s[rb], kr[j % PFK], qreg[rb][j]);
            }
            if (j + PFK < KK) kr[j % PFK] = ld_k(j + PFK);
            else vr[j + PFK - KK] = ld_v(j + PFK - KK);     // the value loop's first operands
            copy_at(j);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) asm_mfma_drain(s[rb]);
    } else {
#pragma unroll
        for (int p = 0; p < PFV; ++p) vr[p] = ld_v(p);
    }
#pragma unroll
    for (int i = 0; i < KK; ++i) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            if (i == 0) asm_mfma_agpr_nop(o[rb * MT], vr[0], pb[rb][0]);
            else asm_mfma_agpr(o[rb * MT + i % MT], vr[i % PFV], pb[rb][i / MT]);
        }
        if (i + PFV < KK) vr[i % PFV] = ld_v(i + PFV);
        if constexpr (HAVE_S) soft(i);
        copy_at(KK + i);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (HAVE_S) soft_end();
}

// SC: the staged kernel (page ids from the staging layout, per-token scales
// copied into LDS beside each key tile: 64 floats per tile slot).
template <int D, bool SC>
__global__ __launch_bounds__(XCfg<D>::THREADS, XCfg<D>::MINB) void extend_kernel(ExtendArgs a) {
    using C = XCfg<D>;
    constexpr int NRB = C::NRB;
    constexpr int SC_BYTES = SC ? 2 * 64 * 4 : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS + SC_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    // grid (Hkv, row blocks, B): dispatch walks x fastest, then y, then z, so
    // the workgroups start heaviest first (longest-processing-time order): the
    // sequence of rank z in decreasing kv end (prefix + chunk; ties by index)
    // with its row blocks from the last (longest kv range) down.  Up to
    // kRankedSeqs sequences are ranked; beyond that they run in index order.
    // Sliding layers: every workgroup's kv range is its rows plus the window,
    // so the work is even, and neighbouring row blocks read mostly the same
    // keys.  Workgroup i runs on XCD i mod 8; renumbering gives each XCD a
    // contiguous range of the order above, so those shared keys are re-read
    // from that XCD's L2 instead of once per XCD from memory (sliding launch
    // of the E2B-like stack ~54 -> ~49.5 us).  Full layers keep the plain
    // order: their heaviest-first start needs the heavy sequences spread
    // over every XCD.
    uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    if (a.window > 0) {
        const uint32_t n = gridDim.x * gridDim.y * gridDim.z;
        const uint32_t i = bx + gridDim.x * (by + gridDim.y * bz);
        const uint32_t per = (n + 7) / 8, tall = (n % 8) ? n % 8 : 8;   // XCDs holding `per`, the rest per - 1
        const uint32_t x = i % 8, k = i / 8;
        const uint32_t v = (x < tall) ? x * per + k : tall * per + (x - tall) * (per - 1) + k;
        bx = v % gridDim.x;
        by = (v / gridDim.x) % gridDim.y;
        bz = v / (gridDim.x * gridDim.y);
    }
    const int32_t g = bx;
    const int32_t blk = gridDim.y - 1 - by;
    int32_t b = bz;
    const int32_t B = gridDim.z;
    if (B > 1 && B <= kRankedSeqs) {
        __shared__ int32_t s_key[kRankedSeqs];
        __shared__ int32_t s_seq;
        if (tid < B) s_key[tid] = min(a.cu_q[tid + 1] - a.cu_q[tid], a.max_q_len) + a.prefix_lens[tid];
        __syncthreads();
        if (tid < B) {
            const int32_t key = s_key[tid];
            int32_t rank = 0;
            for (int32_t j = 0; j < B; ++j) {
                const int32_t kj = s_key[j];
                rank += (kj > key) || (kj == key && j < tid);
            }
            if (rank == (int32_t)bz) s_seq = tid;
        }
        __syncthreads();
        b = s_seq;
    }
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

    // this lane's query rows (one per row block: score column) and their
    // visible kv ranges [row_lo, row_hi] (at D = 256 the position and hi - 1:
    // the softmax forms the range); a row block past the chunk is idle
    const int32_t wrow0 = row0 + wave * 32 * NRB;
    const bool wave_live = wrow0 < rows;
    int32_t my_tok[NRB], my_head[NRB], row_lo[NRB], row_hi[NRB], row_r[NRB], w_pmin[NRB], w_pmax[NRB];
    const float inv_g = a.inv_group;
    bool row_ok[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int32_t r0 = wrow0 + 32 * rb;
        const int32_t my_row = r0 + col;
        row_ok[rb] = my_row < rows;
        my_tok[rb] = row_ok[rb] ? my_row / G : 0;
        my_head[rb] = my_row % G;
        const int32_t my_pos = prefix + my_tok[rb];
        if constexpr (D == 256) {               // the softmax forms the range (FRESH)
            row_lo[rb] = prefix + r0 / G;
            row_r[rb] = r0 % G;
            row_hi[rb] = hi - 1;
        } else {
            row_hi[rb] = min(my_pos, hi - 1);
            row_lo[rb] = (a.window > 0) ? my_pos - a.window + 1 : -(1 << 30);
            row_r[rb] = 0;
        }
        // the row block's extreme positions, for the "tile visible to all rows" test
        w_pmin[rb] = prefix + min(n - 1, r0 / G);
        w_pmax[rb] = prefix + min(n - 1, (r0 + 31) / G);
    }

    const int32_t t_begin = (lo / kTile) * kTile;
    const int32_t n_tiles = (hi - t_begin + kTile - 1) / kTile;
    const int32_t page0 = t_begin / 16;

    // page ids of pages page0 + 64c + lane, batch c; missing pages read page 0
    const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
    // staged: sequence b's pages from the tile of its first row's start lie
    // at b * stride (an even count, so a tile's two pages are neighbours)
    const int32_t sg_first = SC ? 2 * (((a.window > 0) ? max(0, prefix - a.window + 1) : 0) / kTile) : 0;
    auto load_ids = [&](int32_t c) -> int32_t {
        const int32_t pg = page0 + 64 * c + (D == 256 ? lane_id_here() : lane);
        if constexpr (SC) {
            const int32_t jj = pg - sg_first;
            return (jj >= 0 && jj < a.stage_stride) ? b * a.stage_stride + jj : 0;
        }
        int32_t ph = -1;
        if (pg < a.max_pages) ph = pt[pg];
        if ((uint32_t)ph < (uint32_t)a.num_pages) return ph;
        // counted once per workgroup, for pages holding visible keys
        if (wave == 0 && 16 * pg < hi && 16 * pg + 16 > lo) note_bad_id(a.bad_ids, kBadIdExtend);
        return 0;
    };
    // ids holds pages [64 c_ids, +64), ids_next the next 64.  Only the K copy
    // reads page ids (V(t) copies the pages K(t) did, a step later), and a
    // tile's two pages never straddle a batch.
    int32_t c_ids = 0;
    int32_t ids = load_ids(0);
    int32_t ids_next = (2 * n_tiles > 64) ? load_ids(1) : 0;
    auto page_id = [&](int32_t rp) -> int32_t { return __builtin_amdgcn_readlane(ids, rp - 64 * c_ids); };
    // moves the window so that it holds page rp (rp grows by two per step)
    auto slide_ids = [&](int32_t rp) {
        if (rp >= 64 * (c_ids + 1)) {
            ids = ids_next;
            ++c_ids;
            if (64 * (c_ids + 1) < 2 * n_tiles) ids_next = load_ids(c_ids + 1);
        }
    };
    // byte offset of a physical page's block of KV head g in either slab
    auto page_off = [&](int32_t ph) -> int64_t { return ((int64_t)ph * a.hkv + g) * C::PAGE; };

    u32x4 qreg[NRB][C::KK];

    const uint32_t lds0 = lds_addr_of(lds);
    auto kslot = [&](int32_t t) -> uint32_t { return lds0 + (t & 1) * C::HALF; };
    auto vslot = [&](int32_t t) -> uint32_t { return lds0 + 2 * C::HALF + (t & 1) * C::HALF; };
    const uint8_t* k_src = reinterpret_cast<const uint8_t*>(a.k_slab);
    const uint8_t* v_src = reinterpret_cast<const uint8_t*>(a.v_slab);
    uint32_t k_voff[C::NI], v_voff;
    copy_offsets<D>(wave, lane, k_voff, v_voff);

    // LDS offsets this lane reads: K row tau(col), granules (2 kk + h) ^ key;
    // the key has four bits, so it moves a granule within its group of 16
    KOffsets<D> k_off;
    {
        const int j = col >> 3, hh = (col >> 2) & 1, i = col & 3;
        const int tk = 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
        k_off.init(tk * C::KROW + ((h ^ k_swz(tk)) * 16));
    }
    const int v_off = col * 32 + ((h ^ ((col >> 3) & 1)) * 16);

    // O^T tiles: row block rb, output tile m at o[rb * MT + m] (OT tiles)
    f32x16 o[C::OT];
#pragma unroll
    for (int m = 0; m < C::OT; ++m) o[m] = f32x16{};
    float m_run[NRB], l_run[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < C::OT; ++m) pin_agpr(o[m]);
    // the zeros were written by the VALU; the value MFMAs (inline asm, so the
    // compiler does not separate them) read the tiles as SrcC
    asm volatile("s_nop 4" ::: "memory");
    auto is_whole = [&](int32_t t0, int rb) -> bool {
        return (t0 + kTile - 1 <= min(w_pmin[rb], hi - 1)) && (a.window == 0 || w_pmax[rb] - a.window + 1 <= t0);
    };
    // softmax state per row block; stage k of the softmax of tile t0 for
    // every row block, spread (kSoftGap loop steps apart) over the value
    // product of a step
    f32x16 s[NRB];
    u32x4 pb[NRB][2];
    SoftRow sr[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) sr[rb].raise = false;
    // SC: the scale slot (in LDS) of the tile being softmaxed
    const float* sc_cur = reinterpret_cast<const float*>(lds + C::LDS);
    auto scale_slot = [&](int32_t tile) {
        return reinterpret_cast<const float*>(lds + C::LDS + (tile & 1) * 256);
    };
    auto soft_stage_all = [&](int stage, int32_t t0) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            softmax_stage<D == 256, SC>(stage, s[rb], sr[rb], t0, is_whole(t0, rb), row_lo[rb], row_hi[rb], a.window,
                                        h, a.score_scale, m_run[rb], l_run[rb], pb[rb][0], sc_cur, row_r[rb], inv_g);
    };
    auto soft_pack_hi = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) softmax_pack_hi<SC>(s[rb], pb[rb][1], sc_cur);
    };
    // SC: the scales of tile T's pages into its slot, copied with the tile's
    // keys: its second page is its first's neighbour in the staging layout
    // (staged tiles are whole), so one 256-byte copy by wave 0's first 16
    // lanes.  (A tile past the staged range reads page 0's: masked.)
    auto copy_scales = [&](int32_t T, int32_t pid0) {
        if constexpr (SC) {
            if (wave == 0 && lane < 16)
                dma16_s(a.stage_scales + ((int64_t)g * a.stage_pages + pid0) * 32, (uint32_t)(lane * 16),
                        lds0 + C::LDS + (T & 1) * 256);
        }
    };
    constexpr int kSoftGap = C::KK / 8;
    // the stages fit the value loop, and stage 6 (which overwrites pb[rb][0])
    // comes after the value MFMAs that read it (steps 0 .. MT - 1)
    static_assert(kSoftGap * (kSoftStages - 1) < C::KK && kSoftGap * 6 >= C::MT, "softmax stage placement");
    // O of row block rb times the factor its softmax left, once the value
    // MFMAs that wrote O have landed; before the next value product
    auto apply_rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            if (sr[rb].raise) {
                settle_tiles(o);
#pragma unroll
                for (int m = 0; m < C::MT; ++m) agpr_scale(o[rb * C::MT + m], sr[rb].al);
                sr[rb].raise = false;
            }
        }
    };
    // zeroes V of tokens outside [lo, hi) in V tile t: never-written slots may hold NaN
    auto zero_v_edges = [&](int32_t t) {
        const int32_t t0 = t_begin + t * kTile;
        if (t0 >= lo && t0 + kTile <= hi) return;
        uint8_t* vbuf = lds + 2 * C::HALF + (t & 1) * C::HALF;
        for (int idx = tid; idx < 4 * D; idx += C::THREADS) {
            const int p = idx / (2 * D), d = (idx >> 1) % D, hp = idx & 1;
            const int half = hp ^ ((d >> 3) & 1);
            const int32_t tb = t0 + 16 * p + 8 * half;
            u32x4* gp = reinterpret_cast<u32x4*>(vbuf + p * C::PAGE + d * 32 + hp * 16);
            u32x4 v = *gp;
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int32_t tt = tb + 2 * e;
                const uint32_t keep = ((tt >= lo && tt < hi) ? 0xffffu : 0u) |
                                      ((tt + 1 >= lo && tt + 1 < hi) ? 0xffff0000u : 0u);
                w[e] &= keep;
            }
            *gp = u32x4{w[0], w[1], w[2], w[3]};
        }
        lds_barrier();
    };

    // ---- prologue: K(0), V(0), K(1); scores and softmax of tile 0 ----------------
    // ok0, ok1: page offsets of the latest K tile copied, which the V copy
    // of the next step reuses
    int64_t ok0 = 0, ok1 = 0;
    if (n_tiles > 0) {
        const int64_t o0 = page_off(page_id(0)), o1 = page_off(page_id(1));
        copy_k_run<D>(k_src + o0, k_voff, kslot(0), 0, wave);
        copy_k_run<D>(k_src + o1, k_voff, kslot(0), 1, wave);
        copy_v_run<D>(v_src + o0, v_voff, vslot(0), 0, wave);
        copy_v_run<D>(v_src + o1, v_voff, vslot(0), 1, wave);
        copy_scales(0, page_id(0));
        if (n_tiles > 1) {
            ok0 = page_off(page_id(2));
            ok1 = page_off(page_id(3));
            copy_k_run<D>(k_src + ok0, k_voff, kslot(1), 0, wave);
            copy_k_run<D>(k_src + ok1, k_voff, kslot(1), 1, wave);
            copy_scales(1, page_id(2));
        }
    }
    // Q^T operands, loaded while the first tiles are in flight: lane holds
    // Q[row col of block rb][16 kk + 8 h .. +8]; rows past the chunk read token
    // 0 of the chunk and are never written back
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const uint16_t* qp = a.q + ((int64_t)(q0 + my_tok[rb]) * a.hq + (int64_t)g * G + my_head[rb]) * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) qreg[rb][kk] = *reinterpret_cast<const u32x4*>(qp + 16 * kk);
    }
    if (n_tiles > 0) {
        wait_vm<0>();
        lds_barrier();
        if (wave_live) {
            const uint8_t* kbuf = lds + 0;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                s[rb] = asm_mfma_first(*reinterpret_cast<const u32x4*>(kbuf + k_off(0)), qreg[rb][0]);
#pragma unroll
                for (int kk = 1; kk < C::KK; ++kk)
                    asm_mfma_acc(s[rb], *reinterpret_cast<const u32x4*>(kbuf + k_off(kk)), qreg[rb][kk]);
                asm_mfma_drain(s[rb]);
            }
#pragma unroll
            for (int st = 0; st < kSoftStages; ++st) soft_stage_all(st, t_begin);
            soft_pack_hi();
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) sr[rb].raise = false;   // O is still zero
        }
    }

    // ---- steady state: step t = scores of tile t+1 with values of tile t --------
    // (the last step, values only, is peeled off so that the loop body has one
    // path and the accumulator tiles stay put in the AGPR file)
    for (int32_t t = 0; t + 1 < n_tiles; ++t) {
        wait_vm<0>();              // V(t) and K(t+1), copied during the previous step
        lds_barrier();             // ... for every wave; and K(t), V(t-1) are no longer read
        // copies of this step: V(t+1) into V(t-1)'s slot, K(t+2) into K(t)'s
        const int64_t ov0 = ok0, ov1 = ok1;        // V(t+1): the pages of K(t+1)
        const bool k_next = t + 2 < n_tiles;
        if (k_next) {
            slide_ids(2 * t + 4);
            ok0 = page_off(page_id(2 * t + 4));
            ok1 = page_off(page_id(2 * t + 5));
            copy_scales(t + 2, page_id(2 * t + 4));
        }
        if constexpr (SC) sc_cur = scale_slot(t + 1);
        const uint32_t vs = vslot(t + 1), ks = kslot(t + 2);
        // copy c of this step: run c / NI (V(t+1) pages 0, 1, then K(t+2) pages 0,
        // 1), copy c % NI of it
        auto copy = [&](int c) {
            const int j = c / C::NI, i = c % C::NI;
            if (j == 0) copy_piece<D>(false, i, v_src + ov0, k_voff, v_voff, vs, 0, wave);
            else if (j == 1) copy_piece<D>(false, i, v_src + ov1, k_voff, v_voff, vs, 1, wave);
            else if (j == 2) copy_piece<D>(true, i, k_src + ok0, k_voff, v_voff, ks, 0, wave);
            else copy_piece<D>(true, i, k_src + ok1, k_voff, v_voff, ks, 1, wave);
        };
        const int n_copies = (k_next ? 4 : 2) * C::NI;
        zero_v_edges(t);
        if (wave_live) {
            const uint8_t* kbuf = lds + ((t + 1) & 1) * C::HALF;
            const uint8_t* vbuf = lds + 2 * C::HALF + (t & 1) * C::HALF;
            const int32_t t_next = t_begin + (t + 1) * kTile;
            apply_rescale();
            step_mfma<D, true>(
                kbuf, vbuf, k_off, v_off, qreg, pb, s, o, n_copies, copy,
                [&](int k) {
                    if (k % kSoftGap == 0 && k / kSoftGap < kSoftStages) soft_stage_all(k / kSoftGap, t_next);
                },
                soft_pack_hi);
        } else {
            for (int j = 0; j < n_copies; ++j) copy(j);     // a wavefront with no rows still copies its share
        }
#pragma unroll
        for (int m = 0; m < C::OT; ++m) pin_agpr(o[m]);
    }
    if (n_tiles > 0) {
        const int32_t t = n_tiles - 1;
        wait_vm<0>();
        lds_barrier();
        zero_v_edges(t);
        if (wave_live) {
            const uint8_t* vbuf = lds + 2 * C::HALF + (t & 1) * C::HALF;
            apply_rescale();
            step_mfma<D, false>(lds, vbuf, k_off, v_off, qreg, pb, s, o, 0, [](int) {}, [](int) {}, []() {});
        }
        settle_tiles(o);   // the last value MFMAs have landed before the output reads them
    }

    // ---- output: O / l as bf16, through LDS so that every store is a whole row
    // (or two) of 16-byte lanes.  Row r of the workgroup sits at r * 2D bytes,
    // its 16-byte granule q at granule q ^ (r mod D/8) (the 32 rows a
    // wavefront writes at once land in different banks).
    wait_vm<0>();   // no copy is still landing in LDS
    lds_barrier();  // ... and every wavefront is done with the rings
    constexpr int RB = 2 * D, GM = D / 8 - 1;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const float l_tot = sum_halves(l_run[rb]);
        if (!wave_live) continue;
        const float inv = row_ok[rb] ? 1.0f / l_tot : 0.0f;
        const int r = wave * 32 * NRB + 32 * rb + col;
        uint8_t* rowp = lds + r * RB;
#pragma unroll
        for (int m = 0; m < C::MT; ++m) {
            const f32x16& om = o[rb * C::MT + m];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = 4 * m + j;         // granule of dims 32m + 8j .. +8
                *reinterpret_cast<u32x2*>(rowp + ((q ^ (r & GM)) << 4) + 8 * h) =
                    u32x2{cvt_pk_bf16(om[4 * j] * inv, om[4 * j + 1] * inv),
                          cvt_pk_bf16(om[4 * j + 2] * inv, om[4 * j + 3] * inv)};
            }
        }
    }
    lds_barrier();
    // The stores are marked device-coherent and non-temporal (sc1 nt): the
    // output is not read again by this launch, and stores that pass through
    // the XCD's L2 push out the keys and values its other row blocks still
    // read (the sliding launch reads each key once per row block whose window
    // covers it, 34 times at W 512).  Measured: sliding launch 1.43 -> 1.35
    // ms per 28 layers, full 2.95 -> 2.82 ms per 7 (A/B on one box, twice).
    // (A store with more than 8 bytes of data reads its registers after it
    // issues: the s_nop keeps the next instruction off them.)
    const int32_t n_rows = min(C::ROWS, rows - row0);
    // D = 256: the group size through an empty asm, so that the division
    // below forms its reciprocal here instead of keeping the prologue's
    int32_t Go = G;
    if constexpr (D == 256) asm volatile("" : "+s"(Go));
    for (int idx = tid; idx < n_rows * (D / 8); idx += C::THREADS) {
        const int r = idx / (D / 8), q = idx % (D / 8);
        const int32_t row = row0 + r;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * RB + ((q ^ (r & GM)) << 4));
        uint16_t* op = a.out + ((int64_t)(q0 + row / Go) * a.hq + (int64_t)g * Go + row % Go) * D + 8 * q;
        asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(op), "v"(v) : "memory");
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
    a.bad_ids = debug_bad_ids_ptr();
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
    a.inv_group = 1.0f / (float)a.group;
    const bool sc = s.stage_stride > 0;          // a staged call: scales beside the staged pages
    a.stage_scales = sc ? s.slab.k_scale : nullptr;
    a.stage_stride = s.stage_stride;
    a.stage_pages = sc ? s.slab.num_pages : 0;
    const int64_t rows = (int64_t)s.max_q_len * a.group;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.head_dim == 256) {
        using C = XCfg<256>;
        const dim3 grid(s.hkv, (unsigned)((rows + C::ROWS - 1) / C::ROWS), s.num_seqs);
        if (sc) launch(PAKV_TIME_EXTEND, extend_kernel<256, true>, grid, dim3(C::THREADS), 0, st, a);
        else launch(PAKV_TIME_EXTEND, extend_kernel<256, false>, grid, dim3(C::THREADS), 0, st, a);
    } else {
        using C = XCfg<512>;
        const dim3 grid(s.hkv, (unsigned)((rows + C::ROWS - 1) / C::ROWS), s.num_seqs);
        if (sc) launch(PAKV_TIME_EXTEND, extend_kernel<512, true>, grid, dim3(C::THREADS), 0, st, a);
        else launch(PAKV_TIME_EXTEND, extend_kernel<512, false>, grid, dim3(C::THREADS), 0, st, a);
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
