// Staging for the bf16 extend kernel: the layers whose keys and values it
// cannot copy from a slab as they lie -- 8-bit per-token-head codes (int8,
// fp8 E4M3) with their scales, K=V layers (values derived from the stored
// keys), and chunks whose own keys and values come as packed rows beside the
// cache (FreeToken PR #898, description, fourth bullet: the extend kernel
// takes the current chunk from k_extend / v_extend and the prefix from the
// cache; the 8-bit bullet: the scales are read through the same layer
// mapping).  One pass writes, for every page of a call's visible key range,
// what the bf16 kernel reads from a bf16 slab -- a K page (16 rows of D bf16)
// and a dim-major V page (D rows of 16 tokens) -- plus a key scale and a
// value scale per token, into the caller's workspace; the bf16 kernel then
// runs on it, multiplying each score by its key's scale and each weight by
// its key's value scale.  The arithmetic is the general kernel's:
//   - 8-bit codes become bf16 exactly (every int8 code and every finite E4M3
//     code is a bf16 value); the scales stay float32, apart from the codes;
//   - a packed chunk row (positions >= prefix_lens[b]) is copied as given,
//     with scales 1;
//   - a K=V layer's value row is its key row, with value scale
//     1 / sqrt(mean of the row's squares + eps) (unsloth commit 749fb75: the
//     values are the unscaled RMS-normalised keys);
//   - positions outside the range any row of the chunk sees are staged as
//     zeros with zero scales, so a never-written slot (possibly NaN) never
//     reaches the arithmetic; pages past the last row's end get zero scales
//     only (their K and V are masked and zeroed by the kernel).
// Layout: sequence b's staged pages are workspace pages b * stride + j, page
// j holding positions 16 (2 (lo_b / 32) + j) .. + 15, where lo_b is the first
// position its first row sees (0 on a full layer): whole 32-key tiles of the
// bf16 kernel, so a tile's two pages are neighbours (stride is even).  K and
// V blocks (page, KV head) as in a slab; the scales per (KV head, page), the
// 16 key scales then the 16 value scales of its tokens, so that a tile's are
// 256 contiguous bytes.

#include <algorithm>

#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

constexpr int kFmtBF16 = 0, kFmtINT8 = 1, kFmtFP8 = 2, kFmtKEQV = 3;

struct StageArgs {
    const uint8_t* k_slab;
    const uint8_t* v_slab;
    const float* k_scale;
    const float* v_scale;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_q;
    const int32_t* prefix_lens;
    const uint16_t* k_ext;      // packed chunk rows [total_q][Hkv][D] bf16, or null
    const uint16_t* v_ext;      // (null for a K=V layer)
    int32_t max_q_len;
    int32_t max_kv_len;
    int32_t hkv;
    int32_t window;
    int32_t stride;             // staged pages per sequence
    float v_norm_eps;
    uint16_t* sk;               // staged K pages  [B * stride][Hkv][16][D]
    uint16_t* sv;               // staged V pages  [B * stride][Hkv][D][16]
    float* ssc;                 // scales          [Hkv][B * stride][32]: 16 key, 16 value
    uint32_t* bad_ids;          // counters of a PAKV_DEBUG_BOUNDS build, else null
};

template <int F>
__device__ __forceinline__ u32x4 codes8_to_bf16x8(u32x2 w) {
    if constexpr (F == kFmtFP8)
        return u32x4{fp8x2_to_bf16x2(w.x, 0), fp8x2_to_bf16x2(w.x, 2), fp8x2_to_bf16x2(w.y, 0),
                     fp8x2_to_bf16x2(w.y, 2)};
    else
        return u32x4{i8x2_to_bf16x2(w.x, 0), i8x2_to_bf16x2(w.x, 2), i8x2_to_bf16x2(w.y, 0),
                     i8x2_to_bf16x2(w.y, 2)};
}

// Workgroup (page j, KV head g, sequence b): one staged (page, head) block.
template <int D, int F>
__global__ __launch_bounds__(256) void extend_stage_kernel(StageArgs a) {
    constexpr bool Q8 = F == kFmtINT8 || F == kFmtFP8;
    constexpr int ES = Q8 ? 1 : 2;               // bytes per slab element
    constexpr int SEG = D / 16;                  // dims per thread of a key row
    __shared__ __attribute__((aligned(16))) uint16_t kt[16 * D];   // the page's key rows (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t vt[16 * D];   // packed value rows, token-major
    const int tid = threadIdx.x;
    const int32_t j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int32_t q0 = a.cu_q[b];
    const int32_t n = min(a.cu_q[b + 1] - q0, a.max_q_len);
    const int32_t P = a.prefix_lens[b];
    const int32_t hi = min(P + n, a.max_kv_len);                          // the last row's end
    const int32_t lo = (a.window > 0) ? max(0, P - a.window + 1) : 0;     // the first row's start
    const int32_t pg = 2 * (lo / 32) + j;
    const int64_t sblk = ((int64_t)b * a.stride + j) * a.hkv + g;
    float* ssc = a.ssc + ((int64_t)g * gridDim.z * a.stride + (int64_t)b * a.stride + j) * 32;
    // a page no row reads (past the last row's end, or of a sequence with no
    // rows): its K and V are never staged, but its scales are zeros, so that
    // every scale the kernel can meet is finite (a masked key's weight, 0,
    // times its value scale is then 0)
    if (n <= 0 || 16 * pg >= hi) {
        if (tid < 32) ssc[tid] = 0.f;
        return;
    }
    const bool packed = a.k_ext != nullptr;

    // the slab block of this page (read only for live tokens below the chunk
    // when packed); an id outside the pool reads page 0, as the kernels do
    auto slab_blk = [&]() -> int64_t {
        int32_t ph = pg < a.max_pages ? a.page_table[(int64_t)b * a.max_pages + pg] : -1;
        if ((uint32_t)ph >= (uint32_t)a.num_pages) {
            if (tid == 0) note_bad_id(a.bad_ids, kBadIdExtend);
            ph = 0;
        }
        return (int64_t)ph * a.hkv + g;
    };
    const int32_t first_ext = packed ? P : (1 << 30);    // positions from the packed rows
    const bool any_slab = 16 * pg < first_ext;
    const int64_t blk = any_slab ? slab_blk() : 0;

    // ---- keys: thread = (token tt, 8 dims at seg + 128 c for c < SEG / 8), so
    // that the 16 threads of a row read and write 128 / 256 contiguous bytes
    // per instruction ---------------------------------------------------------
    {
        const int tt = tid >> 4, seg = (tid & 15) * 8;
        const int32_t pos = 16 * pg + tt;
        const bool live = pos >= lo && pos < hi;
        const bool ext = pos >= first_ext;
        uint16_t* dst = a.sk + (sblk * 16 + tt) * D + seg;
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < SEG / 8; ++c) {
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (live && ext) {
                x = *reinterpret_cast<const u32x4*>(a.k_ext + ((int64_t)(q0 + pos - P) * a.hkv + g) * D + seg +
                                                     128 * c);
            } else if (live) {
                const uint8_t* src = a.k_slab + ((blk * 16 + tt) * D + seg + 128 * c) * ES;
                if constexpr (Q8) x = codes8_to_bf16x8<F>(*reinterpret_cast<const u32x2*>(src));
                else x = *reinterpret_cast<const u32x4*>(src);
            }
            *reinterpret_cast<u32x4*>(dst + 128 * c) = x;
            *reinterpret_cast<u32x4*>(kt + tt * D + seg + 128 * c) = x;
            if constexpr (F == kFmtKEQV) {
#pragma unroll
                for (int w = 0; w < 4; ++w) ss = sq_sum_bf16x2(x[w], ss);
            }
        }
        if constexpr (F == kFmtKEQV) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
        }
        if ((tid & 15) == 0) {
            float ks = 0.f, vs = 0.f;
            if (live) {
                ks = 1.f;
                vs = 1.f;
                if constexpr (Q8) {
                    if (!ext) {
                        ks = a.k_scale[blk * 16 + tt];
                        vs = a.v_scale[blk * 16 + tt];
                    }
                }
                if constexpr (F == kFmtKEQV) vs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.v_norm_eps);
            }
            ssc[tt] = ks;
            ssc[16 + tt] = vs;
        }
    }
    // packed value rows of the page, token-major, for the transpose below
    if (F != kFmtKEQV && packed && 16 * pg + 15 >= first_ext) {
        const int tt = tid >> 4, seg = (tid & 15) * 8;
        const int32_t pos = 16 * pg + tt;
        const bool take = pos >= first_ext && pos >= lo && pos < hi;
#pragma unroll
        for (int c = 0; c < SEG / 8; ++c) {
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (take)
                x = *reinterpret_cast<const u32x4*>(a.v_ext + ((int64_t)(q0 + pos - P) * a.hkv + g) * D + seg +
                                                     128 * c);
            *reinterpret_cast<u32x4*>(vt + tt * D + seg + 128 * c) = x;
        }
    }
    __syncthreads();

    // ---- values, dim-major: thread = dim d (and d + 256 at D = 512) ----------
#pragma unroll
    for (int d = tid; d < D; d += 256) {
        uint16_t v16[16];
        if constexpr (F == kFmtKEQV) {
#pragma unroll
            for (int t = 0; t < 16; ++t) v16[t] = kt[t * D + d];       // zero already where not live
        } else {
            // the slab's dim-major row of d, then the packed tokens over it
            u32x4 lo8 = u32x4{0u, 0u, 0u, 0u}, hi8 = u32x4{0u, 0u, 0u, 0u};
            if (any_slab) {
                const uint8_t* src = a.v_slab + ((blk * D + d) * 16) * ES;
                if constexpr (Q8) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(src);
                    lo8 = codes8_to_bf16x8<F>(u32x2{w.x, w.y});
                    hi8 = codes8_to_bf16x8<F>(u32x2{w.z, w.w});
                } else {
                    lo8 = *reinterpret_cast<const u32x4*>(src);
                    hi8 = *reinterpret_cast<const u32x4*>(src + 16);
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t wd = (t < 8) ? lo8[(t & 7) >> 1] : hi8[(t & 7) >> 1];
                v16[t] = (uint16_t)((t & 1) ? (wd >> 16) : (wd & 0xffffu));
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int32_t pos = 16 * pg + t;
                if (pos < lo || pos >= hi) v16[t] = 0;
                else if (pos >= first_ext) v16[t] = vt[t * D + d];
            }
        }
        u32x4 o0, o1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            o0[w] = (uint32_t)v16[2 * w] | ((uint32_t)v16[2 * w + 1] << 16);
            o1[w] = (uint32_t)v16[8 + 2 * w] | ((uint32_t)v16[8 + 2 * w + 1] << 16);
        }
        uint16_t* dst = a.sv + (sblk * D + d) * 16;
        *reinterpret_cast<u32x4*>(dst) = o0;
        *reinterpret_cast<u32x4*>(dst + 8) = o1;
    }
}

}  // namespace

namespace pakv {

// Staged pages per sequence: the whole 32-key tiles holding the positions any
// row of a chunk of at most max_q_len tokens sees (at most span of them, from
// the first row's start; the first tile may begin 31 positions earlier).
int32_t extend_stage_stride(int32_t window, int32_t max_q_len, int32_t max_kv_len) {
    const int64_t span = window > 0 ? std::min<int64_t>((int64_t)window + max_q_len, max_kv_len) : max_kv_len;
    return (int32_t)(2 * ((span + 30) / 32 + 1));
}

size_t extend_stage_bytes(int32_t num_seqs, int32_t hkv, int32_t head_dim, int32_t window, int32_t max_q_len,
                          int32_t max_kv_len) {
    const int64_t blocks = (int64_t)num_seqs * extend_stage_stride(window, max_q_len, max_kv_len) * hkv;
    auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
    // (one spare block of scales: a copy of a tile's two pages stays inside)
    return (size_t)(2 * al(blocks * 16 * head_dim * 2) + al((blocks + 1) * 32 * 4));
}

int launch_extend_stage(const ExtendLaunch& s, void* workspace, void* stream) {
    StageArgs a;
    a.k_slab = static_cast<const uint8_t*>(s.slab.k);
    a.v_slab = static_cast<const uint8_t*>(s.slab.v);
    a.k_scale = s.slab.k_scale;
    a.v_scale = s.slab.v_scale;
    a.num_pages = s.slab.num_pages;
    a.page_table = s.page_table;
    a.max_pages = s.max_pages;
    a.cu_q = s.cu_q;
    a.prefix_lens = s.prefix_lens;
    a.k_ext = s.k_ext;
    a.v_ext = s.k_eq_v ? nullptr : s.v_ext;
    a.max_q_len = s.max_q_len;
    a.max_kv_len = s.max_kv_len;
    a.hkv = s.hkv;
    a.window = s.window;
    a.stride = extend_stage_stride(s.window, s.max_q_len, s.max_kv_len);
    a.v_norm_eps = s.v_norm_eps;
    const int64_t blocks = (int64_t)s.num_seqs * a.stride * s.hkv;
    auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
    char* w = static_cast<char*>(workspace);
    a.sk = reinterpret_cast<uint16_t*>(w);
    w += al(blocks * 16 * s.head_dim * 2);
    a.sv = reinterpret_cast<uint16_t*>(w);
    w += al(blocks * 16 * s.head_dim * 2);
    a.ssc = reinterpret_cast<float*>(w);
    a.bad_ids = debug_bad_ids_ptr();
    const int f = s.k_eq_v                         ? kFmtKEQV
                  : s.kv_dtype == PAKV_KV_INT8_PTH ? kFmtINT8
                  : s.kv_dtype == PAKV_KV_FP8_PTH  ? kFmtFP8
                                                   : kFmtBF16;
    const dim3 grid((unsigned)a.stride, (unsigned)s.hkv, (unsigned)s.num_seqs);
    hipStream_t st = static_cast<hipStream_t>(stream);
#define PAKV_STAGE(DD, FF) launch(PAKV_TIME_STAGE, extend_stage_kernel<DD, FF>, grid, dim3(256), 0, st, a)
    if (s.head_dim == 256) {
        if (f == kFmtINT8) PAKV_STAGE(256, kFmtINT8);
        else if (f == kFmtFP8) PAKV_STAGE(256, kFmtFP8);
        else if (f == kFmtKEQV) PAKV_STAGE(256, kFmtKEQV);
        else PAKV_STAGE(256, kFmtBF16);
    } else {
        if (f == kFmtINT8) PAKV_STAGE(512, kFmtINT8);
        else if (f == kFmtFP8) PAKV_STAGE(512, kFmtFP8);
        else if (f == kFmtKEQV) PAKV_STAGE(512, kFmtKEQV);
        else PAKV_STAGE(512, kFmtBF16);
    }
#undef PAKV_STAGE
    return (int)hipGetLastError();
}

}  // namespace pakv
