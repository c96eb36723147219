// paged_attn_decode: split-KV decode with a deterministic combine.
//
// Pass 1 (partial): one workgroup of 4 wavefronts per (sequence b, KV head g,
// split s).  A split is S consecutive positions, aligned to multiples of S in
// absolute position, so its boundaries depend only on the layer, the host's
// length bound and the sequence's own length.  Each wavefront walks its own
// quarter of the split one 16-token page at a time:
//
//   S^T[16 tokens x 16 heads] = K_page[16 x D] . Q_g^T[D x 16]    (MFMA 16x16x32)
//   online softmax per head column (exp2 domain)
//   O^T[D x 16 heads]        += V_page^T[D x 16] . P^T[16 x 16]   (MFMA 16x16x16)
//
// The G query heads that share KV head g are the 16 MFMA columns (columns >= G
// are zero padding), so every K/V element is read from HBM once per
// (sequence, KV head).  K pages are token-major and feed the first product's A
// operand directly (16-byte loads); V pages are dim-major, so the second
// product's A operand (one dim, four consecutive tokens) is one 8-byte load.
// The four wavefronts then merge their (max, sum, O) through LDS in a fixed
// order and write one partial per split.
//
// Pass 2 (combine): per (b, query head), merge the splits in ascending order:
// M = max_s m_s, O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, rounded to
// bf16.  No atomics touch floating-point data, so results are bit-identical
// run to run.
//
// Masks (unsloth commit ca9dbce, one block mask per regime): the decode query
// sits at position L - 1 (L = kv_lens[b]); keys [lo, L) are visible with
// lo = 0 for a full layer and lo = max(0, L - W) for a sliding one.  Scores of
// other keys are selected to -inf, and their value elements are selected to
// zero before the product (slots that were never written may hold NaN).

#include "device_common.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

constexpr int kWaves = 4;

struct DecodeArgs {
    const uint8_t* k_slab;
    const uint8_t* v_slab;
    const float* k_scale;
    const float* v_scale;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* kv_lens;
    const uint16_t* q;
    uint16_t* out;
    int32_t hq;
    int32_t hkv;
    int32_t group;
    int32_t window;
    float score_scale;      // sm_scale * log2(e)
    int32_t split_tokens;
    int32_t max_splits;
    int32_t max_kv_len;
    float* part_o;          // [B][Hkv][max_splits][G][D]
    float* part_ml;         // [B][Hkv][max_splits][G][2]
};

struct SeqRange {
    int32_t lo, hi, base;   // visible keys [lo, hi); splits start at base
};

__device__ __forceinline__ SeqRange seq_range(const DecodeArgs& a, int32_t b) {
    // lengths above the host bound are clamped so the split count never
    // exceeds the grid (and the workspace) sized from it
    int32_t len = clamp_i32(a.kv_lens[b], 1, a.max_kv_len);
    SeqRange r;
    r.hi = len;
    r.lo = (a.window > 0 && len > a.window) ? len - a.window : 0;
    r.base = (r.lo / a.split_tokens) * a.split_tokens;
    return r;
}

// K rows of one page for the first product: lane l reads token l % 16, dims
// 32*kk + 8*(l/16) .. +8.  int8 codes are widened to bf16 exactly.
template <int D, bool INT8>
__device__ __forceinline__ void load_k_page(const uint8_t* kpage, int lane, u32x4 (&kreg)[D / 32]) {
    const int r = lane & 15, qg = lane >> 4;
    if constexpr (!INT8) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(kpage) + r * D + 8 * qg;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) kreg[kk] = *reinterpret_cast<const u32x4*>(p + 32 * kk);
    } else {
        const int8_t* p = reinterpret_cast<const int8_t*>(kpage) + r * D + 8 * qg;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            u32x2 w = *reinterpret_cast<const u32x2*>(p + 32 * kk);
            kreg[kk] = u32x4{i8x2_to_bf16x2(w.x, 0), i8x2_to_bf16x2(w.x, 2),
                             i8x2_to_bf16x2(w.y, 0), i8x2_to_bf16x2(w.y, 2)};
        }
    }
}

// V^T operand of dim tile m: lane l reads dim 16*m + l % 16, tokens
// 4*(l/16) .. +3 of the page (dim-major page: 16 tokens per dim).
template <int D, bool INT8>
__device__ __forceinline__ u32x2 load_v_tile(const uint8_t* vpage, int lane, int m) {
    const int d = 16 * m + (lane & 15), qg = lane >> 4;
    if constexpr (!INT8) {
        return *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(vpage) + d * kPage + 4 * qg);
    } else {
        uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const int8_t*>(vpage) + d * kPage + 4 * qg);
        return u32x2{i8x2_to_bf16x2(w, 0), i8x2_to_bf16x2(w, 2)};
    }
}

template <int D, bool INT8>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
    constexpr int KK = D / 32;   // contraction steps of the first product
    constexpr int MT = D / 16;   // dim tiles of the second product
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int qg = lane >> 4;            // 4-row group of the MFMA layouts
    const int col = lane & 15;           // head column
    const int32_t s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int32_t G = a.group;

    const SeqRange R = seq_range(a, b);
    const int32_t split_start = R.base + s * a.split_tokens;
    if (split_start >= R.hi) return;     // the combine never reads this split
    const int32_t split_end = min(split_start + a.split_tokens, R.hi);
    const int32_t per_wave = a.split_tokens / kWaves;
    const int32_t w_start = max(split_start + wave * per_wave, R.lo);
    const int32_t w_end = min(split_start + (wave + 1) * per_wave, split_end);

    // Q^T operand: column `col` = head g*G + col, dims 32*kk + 8*qg .. +8.
    u32x4 qreg[KK];
    {
        const bool real = col < G;
        const uint16_t* qp = a.q + ((int64_t)b * a.hq + (int64_t)g * G + (real ? col : 0)) * D + 8 * qg;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[kk] = real ? *reinterpret_cast<const u32x4*>(qp + 32 * kk) : u32x4{0, 0, 0, 0};
    }

    f32x4 o[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.0f;

    const int64_t head_block = (int64_t)kPage * D * (INT8 ? 1 : 2);
    for (int32_t t0 = (w_start >> 4) << 4; t0 < w_end; t0 += kPage) {
        const int32_t phys = a.page_table[(int64_t)b * a.max_pages + (t0 >> 4)];
        if ((uint32_t)phys >= (uint32_t)a.num_pages) continue;
        const int64_t blk = ((int64_t)phys * a.hkv + g) * head_block;
        const uint8_t* kpage = a.k_slab + blk;
        const uint8_t* vpage = a.v_slab + blk;

        u32x4 kreg[KK];
        load_k_page<D, INT8>(kpage, lane, kreg);
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) st = mfma_16x16x32(kreg[kk], qreg[kk], st);

        // st[i] = score of token t0 + 4*qg + i for head column `col`
        float ks[4] = {1.f, 1.f, 1.f, 1.f}, vs[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (INT8) {
            const int64_t sb = ((int64_t)phys * a.hkv + g) * kPage + 4 * qg;
            f32x4 k4 = *reinterpret_cast<const f32x4*>(a.k_scale + sb);
            f32x4 v4 = *reinterpret_cast<const f32x4*>(a.v_scale + sb);
            ks[0] = k4.x; ks[1] = k4.y; ks[2] = k4.z; ks[3] = k4.w;
            vs[0] = v4.x; vs[1] = v4.y; vs[2] = v4.z; vs[3] = v4.w;
        }
        float sc[4];
        bool valid[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t t = t0 + 4 * qg + i;
            valid[i] = (t >= w_start) && (t < w_end);
            sc[i] = valid[i] ? st[i] * ks[i] * a.score_scale : -INFINITY;
            mx = fmaxf(mx, sc[i]);
        }
        mx = wave_max_across_groups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = exp2f(sc[i] - m_use);
            psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // P^T operand (tokens 4*qg .. +3 of column `col`), value scales folded in.
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = valid[i] ? p[i] * vs[i] : 0.0f;
        const u32x2 pb = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        const bool full_page = (t0 >= w_start) && (t0 + kPage <= w_end);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            u32x2 va = load_v_tile<D, INT8>(vpage, lane, m);
            if (!INT8 && !full_page) {
                // zero value elements of invisible tokens (never-written slots may be NaN)
                va.x = (valid[0] ? (va.x & 0xffffu) : 0u) | (valid[1] ? (va.x & 0xffff0000u) : 0u);
                va.y = (valid[2] ? (va.y & 0xffffu) : 0u) | (valid[3] ? (va.y & 0xffff0000u) : 0u);
            }
            o[m] = o[m] * alpha;
            o[m] = mfma_16x16x16(va, pb, o[m]);
        }
    }

    // ---- merge the four wavefronts (fixed order) ---------------------------
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ f32x4 s_o[16 * (D / 4)];   // [head][D] as float4 groups
    const float l_tot = wave_sum_across_groups(l_run);
    if (qg == 0) {
        s_m[wave][col] = m_run;
        s_l[wave][col] = l_tot;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][col]);
    const float M_use = (M == -INFINITY) ? 0.0f : M;
    const float my_scale = exp2f(m_run - M_use);
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const f32x4 v = o[m] * my_scale;
                f32x4* dst = &s_o[col * (D / 4) + 4 * m + qg];
                *dst = (w == 0) ? v : (*dst + v);
            }
        }
        __syncthreads();
    }
    // the partial: o relative to M (not normalised), M and L = sum of weights
    const int64_t unit = (((int64_t)b * a.hkv + g) * a.max_splits + s) * G;
    for (int idx = threadIdx.x; idx < G * (D / 4); idx += 256) {
        const int h = idx / (D / 4), c4 = idx % (D / 4);
        reinterpret_cast<f32x4*>(a.part_o + (unit + h) * D)[c4] = s_o[h * (D / 4) + c4];
    }
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float Mh = -INFINITY;
        for (int w = 0; w < kWaves; ++w) Mh = fmaxf(Mh, s_m[w][h]);
        const float Mh_use = (Mh == -INFINITY) ? 0.0f : Mh;
        float L = 0.f;
        for (int w = 0; w < kWaves; ++w) L += s_l[w][h] * exp2f(s_m[w][h] - Mh_use);
        a.part_ml[(unit + h) * 2 + 0] = Mh;
        a.part_ml[(unit + h) * 2 + 1] = L;
    }
}

// Pass 2: one workgroup per (sequence, query head); threads own dims.
template <int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    constexpr int DPT = D / 128;   // dims per thread: 2 or 4
    const int32_t h = blockIdx.x, b = blockIdx.y;
    const int32_t G = a.group;
    const int32_t g = h / G, hl = h % G;
    const SeqRange R = seq_range(a, b);
    const int32_t n_splits = (R.hi - R.base + a.split_tokens - 1) / a.split_tokens;
    const int64_t unit0 = ((int64_t)b * a.hkv + g) * a.max_splits;
    float M = -INFINITY;
    for (int32_t s = 0; s < n_splits; ++s) M = fmaxf(M, a.part_ml[((unit0 + s) * G + hl) * 2]);
    const float M_use = (M == -INFINITY) ? 0.0f : M;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    float L = 0.f;
    const int d0 = threadIdx.x * DPT;
    for (int32_t s = 0; s < n_splits; ++s) {
        const int64_t u = (unit0 + s) * G + hl;
        const float w = exp2f(a.part_ml[u * 2] - M_use);
        L += w * a.part_ml[u * 2 + 1];
        const float* po = a.part_o + u * D + d0;
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] += w * po[e];
    }
    const float inv = 1.0f / L;
    uint16_t* op = a.out + ((int64_t)b * a.hq + h) * D + d0;
#pragma unroll
    for (int e = 0; e < DPT; ++e) op[e] = f32_to_bf16_bits(acc[e] * inv);
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
    a.page_table = s.page_table;
    a.max_pages = s.max_pages;
    a.kv_lens = s.kv_lens;
    a.q = s.q;
    a.out = s.out;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.group = s.plan.group;
    a.window = s.window;
    a.score_scale = s.sm_scale * kLog2e;
    a.split_tokens = s.plan.split_tokens;
    a.max_splits = s.plan.max_splits;
    a.max_kv_len = s.max_kv_len;
    a.part_o = s.part_o;
    a.part_ml = s.part_ml;
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid1(s.plan.max_splits, s.hkv, s.num_seqs);
    dim3 grid2(s.hq, s.num_seqs);
    const bool i8 = s.kv_dtype == PAKV_KV_INT8_PTH;
    if (s.head_dim == 256) {
        if (i8) hipLaunchKernelGGL((decode_partial_kernel<256, true>), grid1, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((decode_partial_kernel<256, false>), grid1, dim3(256), 0, st, a);
        hipLaunchKernelGGL(decode_combine_kernel<256>, grid2, dim3(128), 0, st, a);
    } else {
        if (i8) hipLaunchKernelGGL((decode_partial_kernel<512, true>), grid1, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((decode_partial_kernel<512, false>), grid1, dim3(256), 0, st, a);
        hipLaunchKernelGGL(decode_combine_kernel<512>, grid2, dim3(128), 0, st, a);
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
