// paged_kv_store: scatter new K/V rows into a layer's slab.
//
// One wavefront per (token, KV head) row.  bf16 rows are copied bit for bit;
// 8-bit per-token-head rows are encoded in-kernel (the library's reading of
// the per-token-head formats described in FreeToken PR #898, description
// bullet on the 8-bit formats): amax over the row, one IEEE float32 division
// for the scale (amax / 127 for int8, amax / 448 for fp8), one per element,
// then round half to even: to an integer clamped to +-127 (int8), or to the
// nearest OCP E4M3 value, saturating at +-448 (fp8).  A K=V layer (values
// derived from the keys when read) stores its K rows only.
//
// K pages are token-major ([16][D]); V pages are dim-major ([D][16]), so a V
// row lands as D strided 2-byte (or 1-byte) stores.

#include <mutex>

#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

struct StoreArgs {
    uint8_t* k_slab;
    uint8_t* v_slab;
    float* k_scale;
    float* v_scale;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* cu_tokens;
    const int32_t* start_pos;
    const uint16_t* k;
    const uint16_t* v;      // null for a K=V layer: nothing is stored for V
    int32_t num_seqs;
    int32_t total_tokens;
    int32_t hkv;
    uint32_t* bad_ids;      // counters of a PAKV_DEBUG_BOUNDS build, else null
};

// Sequence of token t: the last b with cu_tokens[b] <= t, found by the 64 lanes
// of a wavefront together (each round narrows the range 64-fold).
__device__ __forceinline__ int32_t find_seq(const int32_t* cu, int32_t num_seqs, int32_t t, int lane) {
    int32_t lo = 0, n = num_seqs;           // answer in [lo, lo + n)
    while (n > 1) {
        const int32_t stride = (n + 63) / 64;
        const int32_t idx = lo + lane * stride;
        const bool le = (idx < lo + n) && (cu[idx] <= t);
        const uint64_t m = __ballot(le);
        const int last = m ? 63 - __builtin_clzll(m) : 0;
        const int32_t end = lo + n;
        lo += last * stride;
        n = min(stride, end - lo);
    }
    return lo;
}

// Physical row address of (token t, head h), or false if the row falls outside
// the page table or the pool.
__device__ __forceinline__ bool locate(const StoreArgs& a, int32_t t, int32_t h, int lane,
                                       int64_t& page_head, int32_t& slot) {
    const int32_t b = find_seq(a.cu_tokens, a.num_seqs, t, lane);
    const int32_t pos = a.start_pos[b] + (t - a.cu_tokens[b]);
    const int32_t pg = pos >> 4;
    const int32_t phys = (pos >= 0 && pg < a.max_pages) ? a.page_table[(int64_t)b * a.max_pages + pg] : -1;
    if ((uint32_t)phys >= (uint32_t)a.num_pages) {
        if (lane == 0) note_bad_id(a.bad_ids, kBadIdStore);
        return false;
    }
    page_head = (int64_t)phys * a.hkv + h;
    slot = pos & 15;
    return true;
}

template <int D>
__global__ __launch_bounds__(256) void store_bf16_kernel(StoreArgs a) {
    constexpr int EPL = D / 64;   // elements per lane: 4 or 8
    const int32_t lane = threadIdx.x & 63;
    const int32_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int32_t h = blockIdx.y;
    if (t >= a.total_tokens) return;
    // the row itself does not depend on where it goes: fetch it first
    const int64_t src = ((int64_t)t * a.hkv + h) * D + lane * EPL;
    const bool has_v = a.v != nullptr;
    uint16_t kv[EPL], vv[EPL];
    if constexpr (EPL == 8) {
        *reinterpret_cast<u32x4*>(kv) = *reinterpret_cast<const u32x4*>(a.k + src);
        if (has_v) *reinterpret_cast<u32x4*>(vv) = *reinterpret_cast<const u32x4*>(a.v + src);
    } else {
        *reinterpret_cast<u32x2*>(kv) = *reinterpret_cast<const u32x2*>(a.k + src);
        if (has_v) *reinterpret_cast<u32x2*>(vv) = *reinterpret_cast<const u32x2*>(a.v + src);
    }
    int64_t ph;
    int32_t slot;
    if (!locate(a, t, h, lane, ph, slot)) return;
    uint16_t* kdst = reinterpret_cast<uint16_t*>(a.k_slab) + (ph * kPage + slot) * D + lane * EPL;
    if constexpr (EPL == 8) *reinterpret_cast<u32x4*>(kdst) = *reinterpret_cast<u32x4*>(kv);
    else *reinterpret_cast<u32x2*>(kdst) = *reinterpret_cast<u32x2*>(kv);
    if (!has_v) return;
    uint16_t* vdst = reinterpret_cast<uint16_t*>(a.v_slab) + ph * kPage * D + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) vdst[(lane * EPL + e) * kPage] = vv[e];
}

// Chunk stores (many tokens per sequence): one workgroup per 16 consecutive
// tokens of the flat list and KV head.  The row kernel writes a token's V row
// as D scattered 2-byte stores into the dim-major page; here the 16 rows are
// staged in LDS and, when they fill one page (slots 0 .. 15 of one page, as
// every block does where sequences start and end on page boundaries), each
// dim's 16 values go out as one contiguous 32-byte row.  Other blocks write
// each present token's values one by one, as the row kernel does.
//
// Where the 16 tokens go: a block inside one sequence (the usual case) needs
// the sequence (a 64-way search by wave 0), its start position and at most
// two page-table entries; a block that crosses sequences searches each token
// (lanes 0 .. 15, binary search over cu_tokens).  Rows whose position falls
// outside the page table or the pool are dropped, as in the row kernel.
template <int D>
__global__ __launch_bounds__(256) void store_bf16_pages_kernel(StoreArgs a) {
    constexpr int CPR = D / 8;                 // 16-byte pieces per row
    constexpr int PER_T = 16 * CPR / 256;      // pieces per thread (2 or 4)
    __shared__ int64_t head_of[16];            // phys page * hkv + h, or -1
    __shared__ int32_t slot_of[16];
    __shared__ __attribute__((aligned(16))) uint16_t vs[16 * D];
    const int t = threadIdx.x, lane = t & 63;
    const int32_t t0 = blockIdx.x * 16;
    const int32_t h = blockIdx.y;
    const int32_t nt = min(16, a.total_tokens - t0);
    const bool has_v = a.v != nullptr;
    // the rows themselves do not depend on where they go: fetch them first
    u32x4 kr[PER_T], vr[PER_T];
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int idx = t + 256 * i, j = idx / CPR, c = idx % CPR;
        const int64_t src = ((int64_t)(t0 + j) * a.hkv + h) * D + c * 8;
        if (j < nt) {
            kr[i] = *reinterpret_cast<const u32x4*>(a.k + src);
            if (has_v) vr[i] = *reinterpret_cast<const u32x4*>(a.v + src);
        }
    }
    if (t < 64) {
        const int32_t b = find_seq(a.cu_tokens, a.num_seqs, t0, lane);
        const int32_t cb = a.cu_tokens[b], ce = a.cu_tokens[b + 1];
        const bool one_seq = t0 + nt <= ce;     // every token of the block is in sequence b
        int32_t bj = b, rel = t0 + lane - cb;
        if (!one_seq && lane < nt) {
            int32_t lo = 0, hi = a.num_seqs - 1;  // the last sequence with cu <= token
            const int32_t tok = t0 + lane;
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (a.cu_tokens[mid] <= tok) lo = mid; else hi = mid - 1;
            }
            bj = lo;
            rel = tok - a.cu_tokens[lo];
        }
        if (lane < 16) {
            int64_t ph = -1;
            int32_t slot = 0;
            if (lane < nt) {
                const int32_t pos = a.start_pos[bj] + rel;
                const int32_t pg = pos >> 4;
                const int32_t phys =
                    (pos >= 0 && pg < a.max_pages) ? a.page_table[(int64_t)bj * a.max_pages + pg] : -1;
                if ((uint32_t)phys < (uint32_t)a.num_pages) {
                    ph = (int64_t)phys * a.hkv + h;
                    slot = pos & 15;
                } else {
                    note_bad_id(a.bad_ids, kBadIdStore);
                }
            }
            head_of[lane] = ph;
            slot_of[lane] = slot;
        }
    }
    if (has_v) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int idx = t + 256 * i, j = idx / CPR;
            if (j < nt) *reinterpret_cast<u32x4*>(vs + idx * 8) = vr[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int idx = t + 256 * i, j = idx / CPR, c = idx % CPR;
        if (j < nt && head_of[j] >= 0)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.k_slab) + (head_of[j] * kPage + slot_of[j]) * D +
                                      c * 8) = kr[i];
    }
    if (!has_v) return;
    bool whole = nt == 16 && head_of[0] >= 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) whole = whole && head_of[j] == head_of[0] && slot_of[j] == j;
#pragma unroll
    for (int dd = 0; dd < D / 256; ++dd) {
        const int d = t + 256 * dd;
        uint16_t* vrow = reinterpret_cast<uint16_t*>(a.v_slab) + d * kPage;
        if (whole) {
            uint32_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = (uint32_t)vs[(2 * e) * D + d] | ((uint32_t)vs[(2 * e + 1) * D + d] << 16);
            u32x4* dst = reinterpret_cast<u32x4*>(vrow + head_of[0] * kPage * D);
            dst[0] = u32x4{w[0], w[1], w[2], w[3]};
            dst[1] = u32x4{w[4], w[5], w[6], w[7]};
        } else {
            for (int j = 0; j < nt; ++j)
                if (head_of[j] >= 0) vrow[head_of[j] * kPage * D + slot_of[j]] = vs[j * D + d];
        }
    }
}

// Nearest OCP E4M3 code of y (ties to even mantissa), saturating at +-448:
// below 2^-6 the grid is the multiples of 2^-9 (y * 512 is exact, and a
// result of 8 is the first normal code); above, y = f * 2^e with f in [1, 2)
// keeps rint((f - 1) * 8) as its 3-bit mantissa, carrying into the exponent
// at 8.  Written from the format's definition; v_rndne_f32 rounds half to even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
    int e = (int)((u >> 23) & 0xffu) - 127;
    const float f = __uint_as_float((u & 0x007fffffu) | 0x3f800000u);
    int q = (int)__builtin_rintf((f - 1.0f) * 8.0f);
    if (q == 8) {
        ++e;
        q = 0;
    }
    if (e > 8 || (e == 8 && q > 6)) {
        e = 8;
        q = 6;
    }
    return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)q;
}

// Encodes EPL bf16 values of one lane into 8-bit codes given the row's scale
// (an all-zero row, scale 0, gets zero codes).
template <int EPL, bool FP8>
__device__ __forceinline__ void encode(const float (&x)[EPL], float scale, uint8_t (&code)[EPL]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        if constexpr (FP8) {
            code[e] = scale > 0.0f ? (uint8_t)e4m3_code(x[e] / scale) : (uint8_t)0;
        } else {
            float c = 0.0f;
            if (scale > 0.0f) {
                c = __builtin_rintf(x[e] / scale);
                c = fminf(fmaxf(c, -127.0f), 127.0f);
            }
            code[e] = (uint8_t)(int8_t)(int)c;
        }
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void store_q8_kernel(StoreArgs a) {
    constexpr int EPL = D / 64;
    constexpr float kMax = FP8 ? 448.0f : 127.0f;   // largest code magnitude
    const int32_t lane = threadIdx.x & 63;
    const int32_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int32_t h = blockIdx.y;
    if (t >= a.total_tokens) return;
    const int64_t src = ((int64_t)t * a.hkv + h) * D + lane * EPL;
    float kx[EPL], vx[EPL];
    float kmax = 0.0f, vmax = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kx[e] = bf16_bits_to_f32(a.k[src + e]);
        vx[e] = bf16_bits_to_f32(a.v[src + e]);
        kmax = fmaxf(kmax, fabsf(kx[e]));
        vmax = fmaxf(vmax, fabsf(vx[e]));
    }
    int64_t ph;
    int32_t slot;
    if (!locate(a, t, h, lane, ph, slot)) return;
    kmax = wave_max(kmax);
    vmax = wave_max(vmax);
    const float ks = kmax / kMax;   // IEEE division (no fast-math in this build)
    const float vs = vmax / kMax;
    uint8_t kc[EPL], vc[EPL];
    encode<EPL, FP8>(kx, ks, kc);
    encode<EPL, FP8>(vx, vs, vc);
    uint8_t* kdst = reinterpret_cast<uint8_t*>(a.k_slab) + (ph * kPage + slot) * D + lane * EPL;
    if constexpr (EPL == 8) *reinterpret_cast<u32x2*>(kdst) = *reinterpret_cast<u32x2*>(kc);
    else *reinterpret_cast<uint32_t*>(kdst) = *reinterpret_cast<uint32_t*>(kc);
    uint8_t* vdst = reinterpret_cast<uint8_t*>(a.v_slab) + ph * kPage * D + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) vdst[(lane * EPL + e) * kPage] = vc[e];
    if (lane == 0) {
        a.k_scale[ph * kPage + slot] = ks;
        a.v_scale[ph * kPage + slot] = vs;
    }
}

// Chunk stores of 8-bit rows: one workgroup per 16 consecutive tokens of the
// flat list and KV head, as store_bf16_pages_kernel.  Wavefront w encodes rows
// 4w .. 4w + 3 exactly as the row kernel does (same amax, scale and codes);
// the K codes go straight to their rows, the V codes to LDS, and when the 16
// tokens fill one page each dim's 16 codes leave as one 16-byte dim-major row
// (the row kernel writes D single bytes per token).
template <int D, bool FP8>
__global__ __launch_bounds__(256) void store_q8_pages_kernel(StoreArgs a) {
    constexpr int EPL = D / 64;
    constexpr float kMax = FP8 ? 448.0f : 127.0f;
    __shared__ int64_t head_of[16];            // phys page * hkv + h, or -1
    __shared__ int32_t slot_of[16];
    __shared__ __attribute__((aligned(16))) uint8_t vq[16 * D];   // V codes, token-major
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int32_t t0 = blockIdx.x * 16;
    const int32_t h = blockIdx.y;
    const int32_t nt = min(16, a.total_tokens - t0);
    // the rows of this wavefront, fetched before their places are known
    float kx[4][EPL], vx[4][EPL];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = 4 * wave + r;
        const int64_t src = ((int64_t)(t0 + j) * a.hkv + h) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kx[r][e] = j < nt ? bf16_bits_to_f32(a.k[src + e]) : 0.0f;
            vx[r][e] = j < nt ? bf16_bits_to_f32(a.v[src + e]) : 0.0f;
        }
    }
    if (t < 64) {
        const int32_t b = find_seq(a.cu_tokens, a.num_seqs, t0, lane);
        const int32_t cb = a.cu_tokens[b], ce = a.cu_tokens[b + 1];
        const bool one_seq = t0 + nt <= ce;
        int32_t bj = b, rel = t0 + lane - cb;
        if (!one_seq && lane < nt) {
            int32_t lo = 0, hi = a.num_seqs - 1;
            const int32_t tok = t0 + lane;
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (a.cu_tokens[mid] <= tok) lo = mid; else hi = mid - 1;
            }
            bj = lo;
            rel = tok - a.cu_tokens[lo];
        }
        if (lane < 16) {
            int64_t ph = -1;
            int32_t slot = 0;
            if (lane < nt) {
                const int32_t pos = a.start_pos[bj] + rel;
                const int32_t pg = pos >> 4;
                const int32_t phys =
                    (pos >= 0 && pg < a.max_pages) ? a.page_table[(int64_t)bj * a.max_pages + pg] : -1;
                if ((uint32_t)phys < (uint32_t)a.num_pages) {
                    ph = (int64_t)phys * a.hkv + h;
                    slot = pos & 15;
                } else {
                    note_bad_id(a.bad_ids, kBadIdStore);
                }
            }
            head_of[lane] = ph;
            slot_of[lane] = slot;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = 4 * wave + r;
        float kmax = 0.0f, vmax = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kmax = fmaxf(kmax, fabsf(kx[r][e]));
            vmax = fmaxf(vmax, fabsf(vx[r][e]));
        }
        kmax = wave_max(kmax);
        vmax = wave_max(vmax);
        const float ks = kmax / kMax;   // IEEE division, as the row kernel
        const float vs = vmax / kMax;
        uint8_t kc[EPL], vc[EPL];
        encode<EPL, FP8>(kx[r], ks, kc);
        encode<EPL, FP8>(vx[r], vs, vc);
        if constexpr (EPL == 8) *reinterpret_cast<u32x2*>(vq + j * D + lane * EPL) = *reinterpret_cast<u32x2*>(vc);
        else *reinterpret_cast<uint32_t*>(vq + j * D + lane * EPL) = *reinterpret_cast<uint32_t*>(vc);
        const int64_t ph = head_of[j];
        if (j < nt && ph >= 0) {
            const int32_t slot = slot_of[j];
            uint8_t* kdst = a.k_slab + (ph * kPage + slot) * D + lane * EPL;
            if constexpr (EPL == 8) *reinterpret_cast<u32x2*>(kdst) = *reinterpret_cast<u32x2*>(kc);
            else *reinterpret_cast<uint32_t*>(kdst) = *reinterpret_cast<uint32_t*>(kc);
            if (lane == 0) {
                a.k_scale[ph * kPage + slot] = ks;
                a.v_scale[ph * kPage + slot] = vs;
            }
        }
    }
    __syncthreads();
    bool whole = nt == 16 && head_of[0] >= 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) whole = whole && head_of[j] == head_of[0] && slot_of[j] == j;
#pragma unroll
    for (int dd = 0; dd < D / 256; ++dd) {
        const int d = t + 256 * dd;
        uint8_t* vrow = a.v_slab + d * kPage;
        if (whole) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)vq[(4 * e) * D + d] | ((uint32_t)vq[(4 * e + 1) * D + d] << 8) |
                       ((uint32_t)vq[(4 * e + 2) * D + d] << 16) | ((uint32_t)vq[(4 * e + 3) * D + d] << 24);
            *reinterpret_cast<u32x4*>(vrow + head_of[0] * kPage * D) = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            for (int j = 0; j < nt; ++j)
                if (head_of[j] >= 0) vrow[head_of[j] * kPage * D + slot_of[j]] = vq[j * D + d];
        }
    }
}

__global__ __launch_bounds__(256) void step_positions_kernel(const int32_t* kv_lens, int32_t B, int32_t* cu,
                                                               int32_t* start) {
    const int32_t b = blockIdx.x * 256 + threadIdx.x;
    if (b <= B) cu[b] = b;
    if (b < B) start[b] = kv_lens[b] - 1;
}

// The counters of a PAKV_DEBUG_BOUNDS build (kBadId* kinds), one copy per
// GPU; host code uses the address debug_bad_ids_ptr() takes, never the name.
__device__ __align__(256) uint32_t debug_bad_ids[pakv::kDebugCounters];

}  // namespace

namespace pakv {

uint32_t* debug_bad_ids_ptr() {
#ifdef PAKV_DEBUG_BOUNDS
    static std::mutex mu;
    static uint32_t* per_device[kNoallocMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_bad_ids)) != hipSuccess) return nullptr;
        per_device[dev] = static_cast<uint32_t*>(p);
    }
    return per_device[dev];
#else
    return nullptr;
#endif
}

int debug_bad_ids_read(uint32_t* out, int n) {
    uint32_t* p = debug_bad_ids_ptr();
    if (!p || n < 0 || n > kDebugCounters) return (int)hipErrorInvalidValue;
    if (hipError_t e = hipDeviceSynchronize()) return (int)e;
    return (int)hipMemcpy(out, p, sizeof(uint32_t) * n, hipMemcpyDeviceToHost);
}

int debug_bad_ids_reset() {
    uint32_t* p = debug_bad_ids_ptr();
    if (!p) return (int)hipErrorInvalidValue;
    const uint32_t zeros[kDebugCounters] = {};
    if (hipError_t e = hipDeviceSynchronize()) return (int)e;
    return (int)hipMemcpy(p, zeros, sizeof zeros, hipMemcpyHostToDevice);
}

int launch_step_positions(const int32_t* kv_lens, int32_t B, int32_t* cu, int32_t* start, void* stream) {
    hipLaunchKernelGGL(step_positions_kernel, dim3((B + 256) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       kv_lens, B, cu, start);
    return (int)hipGetLastError();
}

int launch_store(const StoreLaunch& s, void* stream) {
    StoreArgs a;
    a.k_slab = static_cast<uint8_t*>(const_cast<void*>(s.slab.k));
    a.v_slab = static_cast<uint8_t*>(const_cast<void*>(s.slab.v));
    a.k_scale = const_cast<float*>(s.slab.k_scale);
    a.v_scale = const_cast<float*>(s.slab.v_scale);
    a.num_pages = s.slab.num_pages;
    a.page_table = s.page_table;
    a.max_pages = s.max_pages;
    a.cu_tokens = s.cu_tokens;
    a.start_pos = s.start_pos;
    a.k = s.k;
    a.v = s.v;
    a.num_seqs = s.num_seqs;
    a.total_tokens = s.total_tokens;
    a.hkv = s.hkv;
    a.bad_ids = debug_bad_ids_ptr();
    dim3 grid((s.total_tokens + 3) / 4, s.hkv);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int K = PAKV_TIME_STORE;
    if (s.kv_dtype == PAKV_KV_BF16 && s.total_tokens >= 4 * s.num_seqs) {
        // chunks (on average four or more tokens per sequence): whole V pages
        const dim3 pgrid((s.total_tokens + 15) / 16, s.hkv);
        if (s.head_dim == 256) launch(K, store_bf16_pages_kernel<256>, pgrid, dim3(256), 0, st, a);
        else launch(K, store_bf16_pages_kernel<512>, pgrid, dim3(256), 0, st, a);
    } else if (s.kv_dtype == PAKV_KV_BF16) {
        if (s.head_dim == 256) launch(K, store_bf16_kernel<256>, grid, dim3(256), 0, st, a);
        else launch(K, store_bf16_kernel<512>, grid, dim3(256), 0, st, a);
    } else if (s.total_tokens >= 4 * s.num_seqs) {
        // 8-bit chunks: whole V pages of codes
        const dim3 pgrid((s.total_tokens + 15) / 16, s.hkv);
        const bool fp8 = s.kv_dtype == PAKV_KV_FP8_PTH;
        if (s.head_dim == 256) {
            if (fp8) launch(K, store_q8_pages_kernel<256, true>, pgrid, dim3(256), 0, st, a);
            else launch(K, store_q8_pages_kernel<256, false>, pgrid, dim3(256), 0, st, a);
        } else {
            if (fp8) launch(K, store_q8_pages_kernel<512, true>, pgrid, dim3(256), 0, st, a);
            else launch(K, store_q8_pages_kernel<512, false>, pgrid, dim3(256), 0, st, a);
        }
    } else if (s.kv_dtype == PAKV_KV_FP8_PTH) {
        if (s.head_dim == 256) launch(K, store_q8_kernel<256, true>, grid, dim3(256), 0, st, a);
        else launch(K, store_q8_kernel<512, true>, grid, dim3(256), 0, st, a);
    } else {
        if (s.head_dim == 256) launch(K, store_q8_kernel<256, false>, grid, dim3(256), 0, st, a);
        else launch(K, store_q8_kernel<512, false>, grid, dim3(256), 0, st, a);
    }
    return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace pakv
