// paged_attn_extend for the KV formats the bf16 extend kernel does not take:
// 8-bit per-token-head codes (int8, fp8 E4M3) with their scales, K=V layers
// (values derived from the stored keys), and chunks whose own keys and values
// come as packed rows beside the cache (FreeToken PR #898, description,
// fourth bullet: the extend kernel takes the current chunk from k_extend /
// v_extend and the prefix from the cache; the 8-bit bullet: the scales are
// read through the same layer mapping).
//
// One workgroup per (KV head g, sequence b, block of 32 query rows), query
// rows being the (token, head) pairs of the G heads that share g.  The four
// wavefronts share those rows; wavefront w owns a quarter of the head dims in
// both products:
//
//   S^T[32 kv x 32 rows]  partial over the wave's dims (MFMA 32x32x16); the
//                         four partials are summed through LDS in a fixed
//                         order, so every wave holds the same scores
//   online softmax per row (exp2 domain), redundantly in every wave
//   O^T[D/4 x 32 rows]   += V^T . P^T over the wave's output dims
//
// Each tile of at most 32 kv tokens is staged in LDS as bf16 through
// registers: 8-bit codes are turned into bf16 exactly (the scales stay
// separate: the key scale multiplies the score, the value scale the weight,
// so the products see exact codes), packed rows are copied, and the value
// tile, dim-major for the value product, is read as it lies in a slab page or
// transposed from token-major rows (packed values, or the keys of a K=V
// layer).  A K=V layer's value row is its key row times 1 / sqrt(mean square
// + eps), the factor folded into the weight like a value scale.
//
// Tiles never mix sources: the prefix part [lo, P) comes from the slab (tiles
// aligned to pages), the chunk part [max(P, lo), hi) from the packed rows.
// Without packed rows every tile comes from the slab.  Tokens outside the
// workgroup's visible range are staged as zeros, so slots that were never
// written (possibly NaN) never reach the arithmetic.
//
// Masks (unsloth commit ca9dbce; pegainfer issue #807): the query at position
// p sees key j iff j <= p and, on a sliding layer, p - j < W.

#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kFmtBF16 = 0, kFmtINT8 = 1, kFmtFP8 = 2, kFmtKEQV = 3;
constexpr int kT = 32;          // kv tokens per tile
constexpr int kRows = 32;       // query rows per workgroup

struct GenArgs {
    const uint8_t* k_slab;
    const uint8_t* v_slab;
    const float* k_scale;
    const float* v_scale;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_q;
    const int32_t* prefix_lens;
    const uint16_t* q;
    const uint16_t* k_ext;      // packed chunk rows [total_q][Hkv][D] bf16, or null
    const uint16_t* v_ext;      // (null for a K=V layer)
    uint16_t* out;
    int32_t max_q_len;
    int32_t max_kv_len;
    int32_t hq;
    int32_t hkv;
    int32_t group;
    int32_t window;
    float score_scale;          // sm_scale * log2(e)
    float v_norm_eps;
    uint32_t* bad_ids;          // counters of a PAKV_DEBUG_BOUNDS build, else null
};

template <int D, int F>
struct GCfg {
    static constexpr bool Q8 = F == kFmtINT8 || F == kFmtFP8;
    static constexpr int ES = Q8 ? 1 : 2;            // bytes per slab code
    static constexpr int KP = D * 2 + 16;            // LDS pitch of a staged key row (bf16)
    static constexpr int VP = kT * 2 + 16;           // LDS pitch of a staged value dim
    static constexpr int KL = kT * KP;
    static constexpr int VL = D * VP;
    static constexpr int SX = 4 * 64 * 16 * 4;       // partial scores of the four waves
    static constexpr int LDS = KL + VL + SX + 2 * kT * 4;
    static constexpr int DQ = D / 4;                 // dims per wave
    static constexpr int KK = DQ / 16;               // score MFMAs per tile
    static constexpr int MT = DQ / 32;               // output tiles per wave
    static constexpr int SEG = D / 8;                // dims per thread when a key row is staged
};

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Eight 8-bit codes (two words) -> eight bf16 (exact).
template <int F>
__device__ __forceinline__ u32x4 codes8_to_bf16(u32x2 w) {
    if constexpr (F == kFmtFP8)
        return u32x4{fp8x2_to_bf16x2(w.x, 0), fp8x2_to_bf16x2(w.x, 2), fp8x2_to_bf16x2(w.y, 0),
                     fp8x2_to_bf16x2(w.y, 2)};
    else
        return u32x4{i8x2_to_bf16x2(w.x, 0), i8x2_to_bf16x2(w.x, 2), i8x2_to_bf16x2(w.y, 0),
                     i8x2_to_bf16x2(w.y, 2)};
}

// 8 x 8 transpose of bf16: in[i] holds 8 values of row i; out[j] holds value j
// of rows 0..7.
__device__ __forceinline__ void transpose8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;   // high or low halves of two words
#pragma unroll
        for (int w = 0; w < 4; ++w)
            out[j][w] = __builtin_amdgcn_perm(in[2 * w + 1][j >> 1], in[2 * w][j >> 1], sel);
    }
}

__device__ __forceinline__ float swap_halves_max(float x) {
    float lo = x, hi = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float swap_halves_sum(float x) {
    float lo = x, hi = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
    return lo + hi;
}

template <int D, int F>
__global__ __launch_bounds__(256, (D == 256 ? 2 : 1)) void extend_general_kernel(GenArgs a) {
    using C = GCfg<D, F>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
    uint8_t* kl = lds;                                        // [32 tokens][KP]
    uint8_t* vl = lds + C::KL;                                // [D dims][VP]
    float* sxp = reinterpret_cast<float*>(lds + C::KL + C::VL);
    float* ksc = sxp + 4 * 64 * 16;                           // key scale per staged token
    float* vsc = ksc + kT;                                    // value scale (or K=V factor)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, h = lane >> 5;
    const int32_t g = blockIdx.x;
    const int32_t blk = gridDim.y - 1 - blockIdx.y;
    const int32_t b = blockIdx.z;
    const int32_t G = a.group;
    const int32_t q0 = a.cu_q[b];
    const int32_t n = min(a.cu_q[b + 1] - q0, a.max_q_len);
    const int32_t P = a.prefix_lens[b];
    const int32_t rows = n * G;
    const int32_t row0 = blk * kRows;
    if (n <= 0 || row0 >= rows) return;
    const bool packed = a.k_ext != nullptr;

    const int32_t tok_first = row0 / G;
    const int32_t tok_last = min(n - 1, (row0 + kRows - 1) / G);
    const int32_t hi = min(P + tok_last + 1, a.max_kv_len);
    const int32_t lo = (a.window > 0) ? max(0, P + tok_first - a.window + 1) : 0;

    // this lane's query row (the score column) and its position
    const int32_t my_row = row0 + col;
    const bool row_ok = my_row < rows;
    const int32_t my_tok = row_ok ? my_row / G : 0;
    const int32_t my_head = my_row % G;
    const int32_t my_pos = P + my_tok;
    const int dq = wave * C::DQ;

    // Q^T operand: column my_row, dims dq + 16 kk + 8 h .. +8
    u32x4 qreg[C::KK];
    {
        const uint16_t* qp = a.q + ((int64_t)(q0 + my_tok) * a.hq + (int64_t)g * G + my_head) * D + dq + 8 * h;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4*>(qp + 16 * kk);
    }
    f32x16 o[C::MT];
#pragma unroll
    for (int m = 0; m < C::MT; ++m) o[m] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // key row the lane feeds to the score MFMA: row r = 8 j + 4 hh + i of
    // S^T reads tile token 16 (j / 2) + 8 hh + 4 (j % 2) + i, so the 16 scores
    // a lane receives are tile tokens 8 h .. 8 h + 7 and 16 + 8 h .. + 7: the
    // weights the value MFMA wants from that lane
    const int tau = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);

    const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
    // (called only for pages that hold visible keys)
    auto page_of = [&](int32_t pos) -> int64_t {
        int32_t ph = (pos >> 4) < a.max_pages ? pt[pos >> 4] : -1;
        if ((uint32_t)ph >= (uint32_t)a.num_pages) {
            note_bad_id(a.bad_ids, kBadIdExtend);
            ph = 0;
        }
        return (int64_t)ph * a.hkv + g;      // (page, head) block index
    };

    // tile boundaries: the slab part, then (packed) the chunk part
    const int32_t endA = packed ? min(P, hi) : hi;
    const int32_t startA = (lo / 16) * 16;
    const int32_t nA = endA > startA ? (endA - startA + kT - 1) / kT : 0;
    const int32_t startB = max(P, lo);
    const int32_t nB = (packed && hi > startB) ? (hi - startB + kT - 1) / kT : 0;

    for (int32_t it = 0; it < nA + nB; ++it) {
        const bool from_ext = it >= nA;
        const int32_t t0 = from_ext ? startB + (it - nA) * kT : startA + it * kT;
        const int32_t t_end = from_ext ? min(t0 + kT, hi) : min(t0 + kT, endA);
        const int32_t v_lo = max(t0, lo);     // staged tokens [v_lo, t_end); the rest are zero

        // ---- stage keys: thread = (token tid / 8, dims seg .. seg + SEG) ----
        {
            const int tt = tid >> 3, seg = (tid & 7) * C::SEG;
            const int32_t pos = t0 + tt;
            const bool live = pos >= v_lo && pos < t_end;
            u32x4* dst = reinterpret_cast<u32x4*>(kl + tt * C::KP + seg * 2);
            float ss = 0.f;
            if (live && from_ext) {
                const uint16_t* src = a.k_ext + ((int64_t)(q0 + pos - P) * a.hkv + g) * D + seg;
#pragma unroll
                for (int c = 0; c < C::SEG / 8; ++c) {
                    const u32x4 x = *reinterpret_cast<const u32x4*>(src + 8 * c);
                    dst[c] = x;
                    if constexpr (F == kFmtKEQV) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const float l0 = __uint_as_float(x[w] << 16), h0 = __uint_as_float(x[w] & 0xffff0000u);
                            ss = __builtin_fmaf(l0, l0, __builtin_fmaf(h0, h0, ss));
                        }
                    }
                }
            } else if (live) {
                const int64_t blk_i = page_of(pos);
                const uint8_t* src = a.k_slab + ((blk_i * 16 + (pos & 15)) * D + seg) * C::ES;
#pragma unroll
                for (int c = 0; c < C::SEG / 8; ++c) {
                    u32x4 x;
                    if constexpr (C::Q8) x = codes8_to_bf16<F>(*reinterpret_cast<const u32x2*>(src + 8 * c));
                    else x = *reinterpret_cast<const u32x4*>(src + 16 * c);
                    dst[c] = x;
                    if constexpr (F == kFmtKEQV) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const float l0 = __uint_as_float(x[w] << 16), h0 = __uint_as_float(x[w] & 0xffff0000u);
                            ss = __builtin_fmaf(l0, l0, __builtin_fmaf(h0, h0, ss));
                        }
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < C::SEG / 8; ++c) dst[c] = u32x4{0, 0, 0, 0};
            }
            // per-token factors: thread seg 0 of each token writes them
            if constexpr (F == kFmtKEQV) {
                ss += __shfl_xor(ss, 1, 64);
                ss += __shfl_xor(ss, 2, 64);
                ss += __shfl_xor(ss, 4, 64);
            }
            if ((tid & 7) == 0) {
                float ks = 0.f, vs = 0.f;
                if (live) {
                    ks = 1.f;
                    vs = 1.f;
                    if constexpr (C::Q8) {
                        if (!from_ext) {
                            const int64_t si = page_of(pos) * 16 + (pos & 15);
                            ks = a.k_scale[si];
                            vs = a.v_scale[si];
                        }
                    }
                    if constexpr (F == kFmtKEQV) vs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.v_norm_eps);
                }
                ksc[tt] = ks;
                vsc[tt] = vs;
            }
        }
        // ---- stage values, dim-major -----------------------------------------
        const bool v_token_major = (F == kFmtKEQV) || from_ext;
        if (!v_token_major) {
            // from the slab's dim-major pages: item = (dim d, 8 tokens j8 .. j8+7);
            // the tile starts on a page, so 8 tokens never straddle a page
            for (int item = tid; item < D * (kT / 8); item += 256) {
                const int d = item % D, j8 = (item / D) * 8;
                const int32_t pos = t0 + j8;
                u32x4 x = u32x4{0, 0, 0, 0};
                if (pos + 7 >= v_lo && pos < t_end) {
                    const int64_t blk_i = page_of(pos);
                    const uint8_t* src = a.v_slab + ((blk_i * D + d) * 16 + (pos & 15)) * C::ES;
                    if constexpr (C::Q8) x = codes8_to_bf16<F>(*reinterpret_cast<const u32x2*>(src));
                    else x = *reinterpret_cast<const u32x4*>(src);
                    // tokens of the 8 outside [v_lo, t_end) are zeroed
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int32_t p0 = pos + 2 * w;
                        const uint32_t keep = ((p0 >= v_lo && p0 < t_end) ? 0xffffu : 0u) |
                                              ((p0 + 1 >= v_lo && p0 + 1 < t_end) ? 0xffff0000u : 0u);
                        x[w] &= keep;
                    }
                }
                *reinterpret_cast<u32x4*>(vl + d * C::VP + j8 * 2) = x;
            }
        }
        __syncthreads();
        if (v_token_major) {
            // values from token-major rows, transposed 8 x 8 per thread: the
            // staged keys (K=V) or the packed chunk rows
            for (int item = tid; item < (D / 8) * (kT / 8); item += 256) {
                const int d8 = (item % (D / 8)) * 8, j8 = (item / (D / 8)) * 8;
                u32x4 in[8], tr[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int32_t pos = t0 + j8 + i;
                    if constexpr (F == kFmtKEQV) {
                        in[i] = *reinterpret_cast<const u32x4*>(kl + (j8 + i) * C::KP + d8 * 2);
                    } else {
                        in[i] = u32x4{0, 0, 0, 0};
                        if (pos >= v_lo && pos < t_end)
                            in[i] = *reinterpret_cast<const u32x4*>(a.v_ext + ((int64_t)(q0 + pos - P) * a.hkv + g) * D +
                                                                    d8);
                    }
                }
                transpose8(in, tr);
#pragma unroll
                for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(vl + (d8 + j) * C::VP + j8 * 2) = tr[j];
            }
            __syncthreads();
        }

        // ---- partial scores over this wave's dims --------------------------------
        f32x16 s = f32x16{};
        {
            const uint8_t* kr = kl + tau * C::KP + (dq + 8 * h) * 2;
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) s = mfma32(*reinterpret_cast<const u32x4*>(kr + 32 * kk), qreg[kk], s);
        }
        float* mine = sxp + (wave * 64 + lane) * 16;
#pragma unroll
        for (int e = 0; e < 16; e += 4) *reinterpret_cast<f32x4*>(mine + e) = f32x4{s[e], s[e + 1], s[e + 2], s[e + 3]};
        __syncthreads();
        float sc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float* part = sxp + (w * 64 + lane) * 16;
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(part + e);
                sc[e] += v[0];
                sc[e + 1] += v[1];
                sc[e + 2] += v[2];
                sc[e + 3] += v[3];
            }
        }

        // ---- online softmax of row my_row over tile tokens t0 + tok(e) --------------
        float mx = -INFINITY;
        float vsl[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int tk = (e < 8) ? 8 * h + e : 16 + 8 * h + (e - 8);
            const int32_t pos = t0 + tk;
            const bool vis = row_ok && pos >= v_lo && pos < t_end && pos <= my_pos &&
                             (a.window == 0 || my_pos - pos < a.window);
            sc[e] = vis ? sc[e] * a.score_scale * ksc[tk] : -INFINITY;
            vsl[e] = vsc[tk];
            mx = fmaxf(mx, sc[e]);
        }
        mx = swap_halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_use);
        float psum = 0.f;
        uint32_t pw[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = (sc[e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[e] - m_use);
            const float p1 = (sc[e + 1] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[e + 1] - m_use);
            psum += p0 + p1;
            pw[e / 2] = cvt_pk_bf16(p0 * vsl[e], p1 * vsl[e + 1]);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const u32x4 pb0 = u32x4{pw[0], pw[1], pw[2], pw[3]}, pb1 = u32x4{pw[4], pw[5], pw[6], pw[7]};

        // ---- values: O^T[dims of this wave] += V^T . P^T --------------------------
#pragma unroll
        for (int m = 0; m < C::MT; ++m) {
            o[m] *= alpha;
            const uint8_t* vr = vl + (dq + 32 * m + col) * C::VP + 16 * h;
            o[m] = mfma32(*reinterpret_cast<const u32x4*>(vr), pb0, o[m]);
            o[m] = mfma32(*reinterpret_cast<const u32x4*>(vr + 32), pb1, o[m]);
        }
        __syncthreads();     // the tile's LDS is restaged next
    }

    // ---- output: O^T / l; lane (col, h) holds dims 32 m + 8 e4 + 4 h .. +4 of row col
    const float l_tot = swap_halves_sum(l_run);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    uint16_t* op = a.out + ((int64_t)(q0 + my_tok) * a.hq + (int64_t)g * G + my_head) * D + dq + 4 * h;
#pragma unroll
    for (int m = 0; m < C::MT; ++m) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const f32x16& om = o[m];
            *reinterpret_cast<u32x2*>(op + 32 * m + 8 * e4) =
                u32x2{cvt_pk_bf16(om[4 * e4] * inv, om[4 * e4 + 1] * inv),
                      cvt_pk_bf16(om[4 * e4 + 2] * inv, om[4 * e4 + 3] * inv)};
        }
    }
}

}  // namespace

namespace pakv {

int launch_extend_general(const ExtendLaunch& s, void* stream) {
    GenArgs a;
    a.k_slab = static_cast<const uint8_t*>(s.slab.k);
    a.v_slab = static_cast<const uint8_t*>(s.slab.v);
    a.k_scale = s.slab.k_scale;
    a.v_scale = s.slab.v_scale;
    a.num_pages = s.slab.num_pages;
    a.page_table = s.page_table;
    a.bad_ids = debug_bad_ids_ptr();
    a.max_pages = s.max_pages;
    a.cu_q = s.cu_q;
    a.prefix_lens = s.prefix_lens;
    a.q = s.q;
    a.k_ext = s.k_ext;
    a.v_ext = s.v_ext;
    a.out = s.out;
    a.max_q_len = s.max_q_len;
    a.max_kv_len = s.max_kv_len;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.group = s.hq / s.hkv;
    a.window = s.window;
    a.score_scale = s.sm_scale * kLog2e;
    a.v_norm_eps = s.v_norm_eps;
    const int64_t rows = (int64_t)s.max_q_len * a.group;
    const dim3 grid(s.hkv, (unsigned)((rows + kRows - 1) / kRows), s.num_seqs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int f = s.k_eq_v ? kFmtKEQV
                           : (s.kv_dtype == PAKV_KV_INT8_PTH ? kFmtINT8 : (s.kv_dtype == PAKV_KV_FP8_PTH ? kFmtFP8 : kFmtBF16));
    const int K = PAKV_TIME_EXTEND;
    const dim3 blk(256);
    if (s.head_dim == 256) {
        switch (f) {
            case kFmtINT8: launch(K, extend_general_kernel<256, kFmtINT8>, grid, blk, 0, st, a); break;
            case kFmtFP8: launch(K, extend_general_kernel<256, kFmtFP8>, grid, blk, 0, st, a); break;
            case kFmtKEQV: launch(K, extend_general_kernel<256, kFmtKEQV>, grid, blk, 0, st, a); break;
            default: launch(K, extend_general_kernel<256, kFmtBF16>, grid, blk, 0, st, a); break;
        }
    } else {
        switch (f) {
            case kFmtINT8: launch(K, extend_general_kernel<512, kFmtINT8>, grid, blk, 0, st, a); break;
            case kFmtFP8: launch(K, extend_general_kernel<512, kFmtFP8>, grid, blk, 0, st, a); break;
            case kFmtKEQV: launch(K, extend_general_kernel<512, kFmtKEQV>, grid, blk, 0, st, a); break;
            default: launch(K, extend_general_kernel<512, kFmtBF16>, grid, blk, 0, st, a); break;
        }
    }
    return (int)hipGetLastError();
}

}  // namespace pakv
