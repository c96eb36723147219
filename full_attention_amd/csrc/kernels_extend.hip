// paged_attn_extend: chunked prefill over a paged cache with bf16 MFMA.
//
// One workgroup of 4 wavefronts per (sequence b, KV head g, tile of 64 query
// rows).  Query rows are the (token, head) pairs of the G query heads that
// share KV head g, flattened token-major (row r = token * G + head), so every
// K/V tile staged in LDS serves all heads of the group.  Each wavefront owns
// 16 rows and walks the KV range of the workgroup in 32-token tiles (two pages):
//
//   S^T[32 kv x 16 rows] = K_tile . Q^T          (2 x D/32 MFMA 16x16x32)
//   online softmax per row (exp2 domain)
//   O^T[D x 16 rows]    += V_tile^T . P^T        (D/16 MFMA 16x16x32)
//
// The K sub-tiles take kv tokens in the order 8*(r/4) + 4*j + r%4 (row r of
// sub-tile j), so the scores a lane receives are exactly the 8 consecutive kv
// tokens that the value product's B operand wants in that lane: P never goes
// through LDS.  V pages are dim-major, so the A operand of the value product
// (one dim, 8 consecutive tokens) is a single 16-byte LDS read.
//
// Masks: query row at position p sees kv position j iff j <= p and, on a
// sliding layer, p - j < W (unsloth commit ca9dbce, one block mask per regime;
// pegainfer issue #807, the window counts the query's own position).  Scores
// are selected to -inf; value elements of kv positions outside the
// workgroup's range are zeroed when staged, so never-written slots (possibly
// NaN) contribute nothing.

#include "device_common.h"
#include "launch_timing.h"
#include "pakv_internal.h"

using namespace pakv_dev;

namespace {

constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;
constexpr int kTile = 32;   // kv tokens per staged tile

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

// XOR key of a kv token's K row in LDS: the 16 lanes that read one MFMA A
// operand hit 16 different rows; the key spreads rows over 8 bank groups.
__device__ __forceinline__ int k_swz(int tk) { return ((tk >> 1) & 4) | (tk & 3); }

template <int D>
__global__ __launch_bounds__(256) void extend_kernel(ExtendArgs a) {
    constexpr int KK = D / 32;
    constexpr int MT = D / 16;
    constexpr int CPR = D / 8;           // 16-byte chunks per K row
    __shared__ u32x4 k_lds[kTile * CPR];          // [token][chunk ^ key]
    __shared__ u32x4 v_lds[2 * D * 2];            // [page][dim][half]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int qg = lane >> 4, col = lane & 15;
    const int32_t g = blockIdx.y, b = blockIdx.z;
    const int32_t tile_idx = gridDim.x - 1 - blockIdx.x;   // heaviest tiles first
    const int32_t G = a.group;
    const int32_t q0 = a.cu_q[b];
    const int32_t n = min(a.cu_q[b + 1] - q0, a.max_q_len);
    const int32_t prefix = a.prefix_lens[b];
    const int32_t row0 = tile_idx * kRowsPerWG;
    if (n <= 0 || row0 >= n * G) return;

    const int32_t tok_first = row0 / G;
    const int32_t tok_last = min(n - 1, (row0 + kRowsPerWG - 1) / G);
    const int32_t qpos_min = prefix + tok_first, qpos_max = prefix + tok_last;
    const int32_t hi = min(qpos_max + 1, a.max_kv_len);
    const int32_t lo = (a.window > 0) ? max(0, qpos_min - a.window + 1) : 0;

    // this lane's query row
    const int32_t my_row = row0 + wave * kRowsPerWave + col;
    const int32_t my_tok = my_row / G, my_head = my_row % G;
    const bool row_ok = my_tok < n;
    const int32_t my_pos = prefix + (row_ok ? my_tok : tok_last);

    u32x4 qreg[KK];
    {
        const uint16_t* qp = a.q + ((int64_t)(q0 + (row_ok ? my_tok : 0)) * a.hq + (int64_t)g * G + my_head) * D + 8 * qg;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[kk] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * kk) : u32x4{0, 0, 0, 0};
    }

    f32x4 o[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t head_block = (int64_t)kPage * D;   // elements per (page, head)
    for (int32_t t0 = (lo / kTile) * kTile; t0 < hi; t0 += kTile) {
        // ---- stage K and V of kv tokens [t0, t0 + 32) ------------------------
        int32_t phys[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int32_t pg = (t0 >> 4) + p;
            int32_t ph = -1;
            if (pg < a.max_pages && t0 + 16 * p < hi) ph = a.page_table[(int64_t)b * a.max_pages + pg];
            phys[p] = ((uint32_t)ph < (uint32_t)a.num_pages) ? ph : -1;
        }
#pragma unroll
        for (int j = 0; j < (kTile * CPR) / 256; ++j) {
            const int c = tid + 256 * j;
            const int tk = c / CPR, cr = c % CPR;
            const int p = tk >> 4;
            u32x4 val = u32x4{0, 0, 0, 0};
            if (phys[p] >= 0) {
                const uint16_t* src = a.k_slab + ((int64_t)phys[p] * a.hkv + g) * head_block + (tk & 15) * D + cr * 8;
                val = *reinterpret_cast<const u32x4*>(src);
            }
            k_lds[tk * CPR + (cr ^ k_swz(tk))] = val;
        }
#pragma unroll
        for (int j = 0; j < (2 * D * 2) / 256; ++j) {
            const int c = tid + 256 * j;
            const int p = c / (2 * D), cw = c % (2 * D);
            const int d = cw >> 1, half = cw & 1;
            u32x4 val = u32x4{0, 0, 0, 0};
            if (phys[p] >= 0) {
                const uint16_t* src = a.v_slab + ((int64_t)phys[p] * a.hkv + g) * head_block + d * kPage + half * 8;
                val = *reinterpret_cast<const u32x4*>(src);
                const int32_t tk0 = t0 + 16 * p + 8 * half;
                if (tk0 < lo || tk0 + 8 > hi) {
                    uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int32_t ta = tk0 + 2 * e, tb = ta + 1;
                        const uint32_t keep_lo = (ta >= lo && ta < hi) ? 0xffffu : 0u;
                        const uint32_t keep_hi = (tb >= lo && tb < hi) ? 0xffff0000u : 0u;
                        w[e] &= (keep_lo | keep_hi);
                    }
                    val = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
            v_lds[c] = val;
        }
        __syncthreads();

        // ---- scores -------------------------------------------------------
        f32x4 st[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = col;
            const int tk = 8 * (r >> 2) + 4 * j + (r & 3);
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const u32x4 ka = k_lds[tk * CPR + ((4 * kk + qg) ^ k_swz(tk))];
                acc = mfma_16x16x32(ka, qreg[kk], acc);
            }
            st[j] = acc;
        }
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t kp = t0 + 8 * qg + 4 * j + i;
                const bool vis = (kp <= my_pos) && (a.window == 0 || my_pos - kp < a.window);
                const float v = vis ? st[j][i] * a.score_scale : -INFINITY;
                sc[4 * j + i] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = wave_max_across_groups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[8], psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = exp2f(sc[e] - m_use);
            psum += p[e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const u32x4 pb = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        // ---- values -------------------------------------------------------
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int d = 16 * m + col;
            const u32x4 va = v_lds[((qg >> 1) * D + d) * 2 + (qg & 1)];
            o[m] = o[m] * alpha;
            o[m] = mfma_16x16x32(va, pb, o[m]);
        }
        __syncthreads();
    }

    const float l_tot = wave_sum_across_groups(l_run);
    if (!row_ok) return;
    const float inv = 1.0f / l_tot;
    uint16_t* op = a.out + ((int64_t)(q0 + my_tok) * a.hq + (int64_t)g * G + my_head) * D;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int d = 16 * m + 4 * qg;
        const u32x2 w = u32x2{pack_bf16x2(o[m][0] * inv, o[m][1] * inv), pack_bf16x2(o[m][2] * inv, o[m][3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = w;
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
    dim3 grid((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG), s.hkv, s.num_seqs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.head_dim == 256) launch(PAKV_TIME_EXTEND, extend_kernel<256>, grid, dim3(256), 0, st, a);
    else launch(PAKV_TIME_EXTEND, extend_kernel<512>, grid, dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

}  // namespace pakv
