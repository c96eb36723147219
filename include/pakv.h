/*
 * pakv.h -- paged KV-cache attention with per-layer mask regimes, for MI355X (gfx950).
 *
 * The calls follow how the pages state the problem:
 *  - each layer that owns KV has its own paged cache; a KV-shared layer points at
 *    its source layer's cache instead of holding one (unsloth commit dee9371,
 *    "scripts": shared layers reference the store layer's PagedKVCache);
 *  - one (layer, source) list decides which slab every layer reads, and a shared
 *    layer with no earlier layer of its attention type is refused
 *    (FreeToken PR #898, "perf(gemma4): read the source layer's kv slab on
 *    kv-shared layers", description, first and second bullets, and the review);
 *  - the store returns early for a shared layer, and the extend and decode
 *    kernels find slabs and scales through the same mapping (same PR,
 *    description, fourth and fifth bullets);
 *  - two mask regimes: full layers are purely causal, sliding layers are causal
 *    and keep key j for query p only while p - j < W, so the window counts the
 *    query's own position (unsloth commit ca9dbce, the change that builds one
 *    block mask per attention regime; pegainfer issue #807, Description, on
 *    passing W - 1 to an API that measures an inclusive distance).  This
 *    library takes W itself.
 *
 * Conventions shared by every call:
 *  - No exceptions cross the ABI.  Every call returns a pakv_status; the text of
 *    the last failure on the calling thread is available from pakv_last_error()
 *    until that thread's next call.
 *  - Argument errors are found on the host and returned before anything is
 *    launched.  Nothing is launched either when a call has no work (zero tokens).
 *  - Device pointers are plain device addresses owned by the caller.  The library
 *    never allocates, frees or copies device memory, never synchronises, and
 *    never reads device memory from the host: every call is asynchronous on the
 *    stream it is given (a hipStream_t passed as void*; NULL is the null stream).
 *    The one exception is the pair of page-id diagnostic calls of a
 *    PAKV_DEBUG_BOUNDS build (pakv_debug_bounds_counts / _reset), which wait
 *    for the device and copy their counters.
 *  - bf16 tensors are 16-bit bfloat16 bit patterns.  Page size is 16 tokens.
 *  - Device-side values (lengths, page ids) are clamped into range so that no
 *    access leaves the buffers the descriptors describe: a length above the
 *    stated bound or a page id outside [0, num_pages) never faults, but the
 *    affected outputs are then unspecified.
 *
 * Slab layout (one slab per owning layer; K and V are separate buffers):
 *   K codes : [num_pages][Hkv][16][D]  token-major inside a page
 *   V codes : [num_pages][Hkv][D][16]  dim-major inside a page (each dim's 16
 *             tokens are contiguous), so that the value contraction over tokens
 *             reads contiguous runs
 *   codes are bf16 (2 bytes) for PAKV_KV_BF16, int8 for PAKV_KV_INT8_PTH and
 *   OCP FP8 E4M3 bytes for PAKV_KV_FP8_PTH.
 *   8-bit scales: k_scale, v_scale : float32 [num_pages][Hkv][16], one per
 *   token and KV head (FreeToken PR #898, description bullet on the
 *   per-token-head formats; "End to end": D + 4 bytes per row for either
 *   8-bit format).
 *   A K=V layer (k_eq_v below) has a K slab only: its values are derived from
 *   the stored keys whenever they are read.
 * Every (page, head) block is 16*D codes, contiguous.
 *
 * 8-bit per-token-head encodings (the pages do not print them; this library's
 * reading): for a row x of D bf16 values, amax = max|x_d| and scale =
 * fl32(amax / M) by IEEE float32 division, M = 127 (int8) or 448 (fp8, the
 * largest E4M3 value); y_d = fl32(x_d / scale); int8: code_d =
 * clamp(rne(y_d), -127, 127); fp8: code_d = the E4M3 value nearest y_d, ties
 * to the even mantissa, saturating at +-448.  An all-zero row gets scale 0
 * and zero codes.  A stored element decodes to value(code) * scale.
 */
#ifndef PAKV_H
#define PAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAKV_PAGE_SIZE 16

typedef enum {
    PAKV_OK = 0,
    PAKV_ERR_INVALID = 1,     /* a null pointer, a negative size, an index out of range */
    PAKV_ERR_UNSUPPORTED = 2, /* a shape this build has no kernel for (head_dim, group size, page size) */
    PAKV_ERR_ALIAS = 3,       /* a KV-sharing rule is broken (see pakv_layer_map_create) */
    PAKV_ERR_WORKSPACE = 4,   /* decode or staging workspace missing or too small */
    PAKV_ERR_HIP = 5          /* the HIP runtime reported an error; the message carries its text */
} pakv_status;

typedef enum {
    PAKV_KV_BF16 = 0,     /* bf16 codes */
    PAKV_KV_INT8_PTH = 1, /* int8 codes + one float32 scale per token and KV head */
    PAKV_KV_FP8_PTH = 2   /* fp8 E4M3 codes + one float32 scale per token and KV head */
} pakv_kv_dtype;

/* Per-layer description.
 *   head_dim      : 256 or 512
 *   num_q_heads   : Hq; a multiple of num_kv_heads, with Hq / Hkv <= 16
 *   num_kv_heads  : Hkv >= 1.  Query head h reads KV head h / (Hq / Hkv).
 *   window        : 0 for a full (causal) layer; W > 0 for a sliding layer, where
 *                   key position j is visible to query position p iff
 *                   j <= p and p - j < W.
 *   kv_source     : -1 if the layer owns a slab, else the index of the owning
 *                   layer whose slab it reads.
 *   kv_dtype      : a pakv_kv_dtype.
 *   sm_scale      : softmax scale applied to q.k (for example 1/sqrt(head_dim)).
 *   k_eq_v        : 1 for a layer whose value row is its key row RMS-normalised
 *                   without a learned scale, v = k / sqrt(mean_d k_d^2 +
 *                   v_norm_eps) (unsloth commit 749fb75: attention_k_eq_v on
 *                   the full layers, the value being the key projection
 *                   followed only by a scale-free v_norm; pegainfer issue #807,
 *                   Description, third paragraph: whether K and V can share
 *                   storage).  Such a layer stores and reads its K slab only;
 *                   bf16 layers only in this build.  0 otherwise.
 *   v_norm_eps    : the eps of that norm (k_eq_v layers; e.g. 1e-6). */
typedef struct {
    int32_t head_dim;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t window;
    int32_t kv_source;
    int32_t kv_dtype;
    float sm_scale;
    int32_t k_eq_v;
    float v_norm_eps;
} pakv_layer_desc;

/* Device buffers of one owning layer's slab (layout above).  k_scale / v_scale
 * are NULL for bf16 slabs; v is NULL for a K=V layer.  page_size must be 16. */
typedef struct {
    void* k;
    void* v;
    float* k_scale;
    float* v_scale;
    int32_t num_pages;
    int32_t page_size;
} pakv_slab;

/* Page table shared by the layers of one batch: device int32
 * [num_seqs][max_pages_per_seq]; entry [b][i] is the physical page holding
 * positions 16*i .. 16*i + 15 of sequence b.  Owned by the caller. */
typedef struct {
    const int32_t* page_table;
    int32_t num_seqs;
    int32_t max_pages_per_seq;
} pakv_pages;

typedef struct pakv_layer_map pakv_layer_map;

/* Text of the calling thread's last failure ("" if none).  Valid until the
 * thread's next pakv_* call. */
const char* pakv_last_error(void);

/* Source rule for a model whose layers first_shared .. n_layers-1 are KV-shared
 * (FreeToken PR #898, description, first bullet): such a layer reads the last
 * layer before first_shared with the same layer_type (any int32 tag, for
 * example 0 = sliding, 1 = full).  Layers below first_shared read themselves.
 * Writes out_source[n_layers] (host memory).  first_shared >= n_layers means
 * no sharing.  Returns PAKV_ERR_ALIAS, writing nothing, if a shared layer has
 * no earlier layer of its type (the refusal asked for in that PR's review). */
pakv_status pakv_resolve_kv_sources(int32_t n_layers, const int32_t* layer_type,
                                    int32_t first_shared, int32_t* out_source);

/* Builds the host-side map of n layers from descs (copied; host memory).
 * Returns PAKV_ERR_ALIAS if some kv_source is not an earlier layer, is itself
 * shared, or differs from the layer in head_dim, num_kv_heads, window,
 * kv_dtype, k_eq_v or v_norm_eps; PAKV_ERR_UNSUPPORTED for a head_dim other
 * than 256 / 512, a group size Hq / Hkv above 16 or an 8-bit K=V layer;
 * PAKV_ERR_INVALID for other bad fields.
 * On success *out owns the map; release it with pakv_layer_map_destroy. */
pakv_status pakv_layer_map_create(const pakv_layer_desc* descs, int32_t n, pakv_layer_map** out);
void pakv_layer_map_destroy(pakv_layer_map* map);

/* Attaches a slab to an owning layer (the map keeps the pointers; the caller
 * keeps ownership of the memory).  PAKV_ERR_ALIAS for a shared layer: a shared
 * layer never has a slab of its own.  Rebinding replaces the previous slab. */
pakv_status pakv_layer_map_bind_slab(pakv_layer_map* map, int32_t layer, const pakv_slab* slab);

/* The layer whose slab `layer` reads (itself for an owner). */
pakv_status pakv_layer_map_source(const pakv_layer_map* map, int32_t layer, int32_t* src);

/* KV bytes per token over owning layers only (FreeToken PR #898, description,
 * third bullet: only layers that own KV are priced), split into the full group
 * (window == 0) and the window group: sum of Hkv * 2 * row (Hkv * row for a
 * K=V layer, which stores no V), row = 2*D for bf16 and D + 4 for the 8-bit
 * per-token-head formats. */
pakv_status pakv_kv_bytes_per_token(const pakv_layer_map* map, int64_t* full_bytes, int64_t* window_bytes);

/* Bytes of the K (or V) code buffer and of one scale buffer for a slab of
 * num_pages pages of the given layer (scale bytes are 0 for bf16). */
pakv_status pakv_slab_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_pages,
                            size_t* code_bytes, size_t* scale_bytes);

/* Writes new K/V rows into the slab of `layer`.
 *   cu_tokens   : device int32 [num_seqs + 1], prefix sums; sequence b owns rows
 *                 cu_tokens[b] .. cu_tokens[b+1]-1 of k and v
 *   start_pos   : device int32 [num_seqs]; row i of sequence b goes to position
 *                 start_pos[b] + i
 *   k, v        : device bf16 [total_tokens][Hkv][D], token-major (v is not
 *                 read, and may be NULL, for a K=V layer)
 * For an 8-bit layer the rows are encoded in-kernel (see the header comment).
 * A shared layer returns PAKV_OK and launches nothing: its source stored the
 * same rows earlier in the forward (FreeToken PR #898, description, fourth
 * bullet).  Rows whose position falls outside the page table are dropped. */
pakv_status pakv_paged_kv_store(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                const int32_t* cu_tokens, const int32_t* start_pos,
                                const void* k, const void* v,
                                int32_t num_seqs, int32_t total_tokens, void* stream);

/* Workspace bytes pakv_paged_attn_decode needs for these sizes (enough for
 * pakv_paged_attn_decode_planned as well). */
size_t pakv_decode_workspace_bytes(const pakv_layer_map* map, int32_t layer,
                                   int32_t num_seqs, int32_t max_kv_len);
#define PAKV_DECODE_PLAN_MISMATCH 1u
#define PAKV_DECODE_XCD_SPLIT 2u

/* One decode query per sequence.
 *   kv_lens     : device int32 [num_seqs], tokens stored for the sequence
 *                 including the current one, 1 <= kv_lens[b] <= max_kv_len.
 *                 The query sits at position kv_lens[b] - 1; its own K/V must
 *                 already be stored (by this layer's source for a shared layer).
 *   q, out      : device bf16 [num_seqs][Hq][D]
 *   max_kv_len  : host upper bound on kv_lens (lengths above it are clamped)
 *   workspace   : device memory of at least pakv_decode_workspace_bytes(...),
 *                 zero-filled before its first use; every call leaves it
 *                 zero-filled again (per-sequence arrival counters live there),
 *                 except for its first 32-bit word, the status word below.
 *                 Calls that may overlap need separate workspaces.
 * Status word (workspace bytes 0..3): bits that a call sets when its kernel
 * detects a condition it cannot report through the return value (the kernel
 * runs after the call returns); they stay set until the caller clears them.
 *   PAKV_DECODE_PLAN_MISMATCH : the plan given to a planned or append call was
 *                 made for another num_seqs, Hkv, window or max_kv_len; the
 *                 call then wrote no output and changed nothing else.
 *   PAKV_DECODE_XCD_SPLIT     : some unit merged inside one XCD's L2 had
 *                 workgroups on several XCDs (see pakv_workgroup_xcds); its
 *                 outputs may be wrong.  Checked only while
 *                 pakv_set_decode_checks(PAKV_CHECK_XCD_PLACEMENT) is on.
 * num_seqs must not exceed 1023 and num_seqs * Hkv 8192 (PAKV_ERR_UNSUPPORTED).
 * A shared layer reads its source's slab (and scales) with its own descriptor
 * (window, sm_scale, Hq).  The keys of all sequences form one stream of
 * 16-token pages that a fixed number of workgroups split evenly; partial
 * results are merged in a fixed order, so the output is bit-identical from
 * run to run and does not depend on page placement (it may differ in the last
 * bits when other sequences of the batch change, since they move the split
 * points). */
pakv_status pakv_paged_attn_decode(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                   const int32_t* kv_lens, const void* q, void* out,
                                   int32_t num_seqs, int32_t max_kv_len,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Decode in two calls, for a step that decodes several layers over the same
 * sequences: the split of the keys into workgroup runs and the page ids of
 * every run depend only on kv_lens, the page table, the window and Hkv, so
 * pakv_decode_plan computes them once into `plan` (device memory of at least
 * pakv_decode_plan_bytes(...), owned by the caller; asynchronous on the
 * stream) and pakv_paged_attn_decode_planned runs a layer's attention from it.
 * A plan made for `layer` serves every layer with the same window and Hkv
 * while kv_lens, the page table, num_seqs and max_kv_len stay as they were
 * when it was made.  The kernel checks the plan's header against the call's
 * num_seqs, Hkv, window and max_kv_len: on a mismatch it writes nothing and
 * sets PAKV_DECODE_PLAN_MISMATCH in the workspace's status word.  Changed
 * kv_lens or page table entries under an unchanged header it cannot tell:
 * page ids are re-clamped to the slab, so such a stale plan gives wrong
 * values, never an access outside the slab.  The planned call takes the same arguments and
 * workspace as pakv_paged_attn_decode, minus kv_lens, and gives bit-identical
 * output. */
size_t pakv_decode_plan_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_seqs, int32_t max_kv_len);
pakv_status pakv_decode_plan(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                             const int32_t* kv_lens, int32_t num_seqs, int32_t max_kv_len,
                             void* plan, size_t plan_bytes, void* stream);
pakv_status pakv_paged_attn_decode_planned(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                           const void* plan, size_t plan_bytes, const void* q, void* out,
                                           int32_t num_seqs, int32_t max_kv_len,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* Store, then decode, in one launch: the decode step of a layer whose new K/V
 * row (one token per sequence) has not been stored yet.  The result and the
 * slab afterwards are bit-identical to pakv_paged_kv_store of that row at
 * position kv_lens[b] - 1 (cu_tokens = 0..num_seqs) followed by
 * pakv_paged_attn_decode_planned with the same plan; the row is copied
 * straight into the staged page of the workgroup that reads it, so the store
 * costs no launch and no wait of its own.  (FreeToken PR #898: the store runs
 * before attention in the forward, description, fourth bullet, and a store
 * per layer per step is what its decode benchmark paragraph puts the shared
 * layers' decode gain down to.)
 *   k_new, v_new : device bf16 [num_seqs][Hkv][D], owned by the caller
 *   plan         : from pakv_decode_plan for this step (it carries kv_lens)
 * Other arguments as in pakv_paged_attn_decode_planned; kv_lens[b] must not
 * exceed max_kv_len.  A row whose page id (page_table[b][(kv_lens[b]-1)/16])
 * lies outside [0, num_pages) is not written, as pakv_paged_kv_store drops
 * such rows; the new token is still attended.  A shared layer stores nothing (its source's call stored
 * the row) and k_new/v_new may be NULL: the call is then a planned decode.  An
 * owning layer with 8-bit or K=V storage returns PAKV_ERR_UNSUPPORTED before
 * any launch (call pakv_paged_kv_store, then the planned decode). */
pakv_status pakv_paged_attn_decode_append(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const void* plan, size_t plan_bytes, const void* k_new,
                                          const void* v_new, const void* q, void* out,
                                          int32_t num_seqs, int32_t max_kv_len,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* pakv_paged_attn_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The call allocates nothing: its
 * plan, partials and arrival counters live in a static device array of the
 * library, pakv_decode_noalloc_max_bytes() bytes (64 MiB) on each GPU it runs
 * on, kept until the process ends.  Arguments and output as in
 * pakv_paged_attn_decode (bit-identical results).  A call whose workspace
 * (pakv_decode_workspace_bytes) would exceed that size returns
 * PAKV_ERR_WORKSPACE before any launch.  Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must not be made; calls in one stream are fine.  The
 * array's status word is not readable by the caller. */
pakv_status pakv_paged_attn_decode_noalloc(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                           const int32_t* kv_lens, const void* q, void* out,
                                           int32_t num_seqs, int32_t max_kv_len, void* stream);
size_t pakv_decode_noalloc_max_bytes(void);

/* Chunked prefill: a chunk of new queries per sequence after a cached prefix.
 *   cu_q        : device int32 [num_seqs + 1], prefix sums of chunk lengths n_b
 *   prefix_lens : device int32 [num_seqs]; query i of sequence b sits at
 *                 position prefix_lens[b] + i
 *   q, out      : device bf16 [total_q][Hq][D], token-major, packed by cu_q
 *   max_q_len   : host upper bound on n_b;  max_kv_len : host bound on
 *                 prefix_lens[b] + n_b
 * The chunk's own K/V must already be stored (by the source for a shared layer,
 * as the source runs earlier in the forward); the kernel reads prefix and chunk
 * from the slab.  Every format: bf16 slabs go to an extend kernel built for
 * them; 8-bit and K=V layers to one that stages each tile in bf16 (exact
 * codes, scales applied to the scores and the weights). */
pakv_status pakv_paged_attn_extend(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                   const int32_t* cu_q, const int32_t* prefix_lens,
                                   const void* q, void* out,
                                   int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                   int32_t max_kv_len, void* stream);

/* Chunked prefill with the chunk's own keys and values given as packed rows
 * (FreeToken PR #898, description, fourth bullet: the extend kernel takes the
 * current chunk from k_extend / v_extend, and the attention module passes k, v
 * to the backend even on a shared layer): positions prefix_lens[b] ..
 * prefix_lens[b] + n_b - 1 read k_ext / v_ext, exactly as given in bf16
 * whatever format the slab stores; only the prefix (positions below
 * prefix_lens[b]) is read from the slab.  The call stores nothing: an owning
 * layer's pakv_paged_kv_store of the same rows may come before or after it.
 *   k_ext, v_ext : device bf16 [total_q][Hkv][D], token-major, packed by cu_q
 *                  (for a shared layer, its source's rows); v_ext is not read,
 *                  and may be NULL, for a K=V layer (values from k_ext)
 * Other arguments as in pakv_paged_attn_extend. */
pakv_status pakv_paged_attn_extend_packed(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const int32_t* cu_q, const int32_t* prefix_lens,
                                          const void* q, const void* k_ext, const void* v_ext, void* out,
                                          int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, void* stream);

/* Chunked prefill for every format on the bf16 MFMA kernel.  8-bit slabs, K=V
 * layers and packed chunks (which pakv_paged_attn_extend and _packed run on a
 * kernel that stages each tile itself) are first staged into `workspace` by
 * one pass: for every page of the call's visible key range, the keys as bf16
 * codes (8-bit codes exactly; packed rows as given), the values as bf16
 * dim-major pages (a K=V layer's values are its key rows), and per token a key
 * scale and a value scale (the format's scales; 1 for packed rows; a K=V
 * layer's value scale 1 / sqrt(mean square + eps), unsloth commit 749fb75).
 * The bf16 kernel then reads the staged pages, multiplying each score by its
 * key's scale and each weight by its key's value scale: the arithmetic of the
 * other extend calls, exact codes with float32 scales.  A bf16 layer's own
 * chunk (k_ext NULL) needs no staging and runs as in pakv_paged_attn_extend.
 *   k_ext, v_ext : NULL (the chunk is read from the slab, as in
 *                  pakv_paged_attn_extend), or the packed chunk rows as in
 *                  pakv_paged_attn_extend_packed
 *   workspace    : device memory of at least pakv_extend_staging_bytes(...,
 *                  packed = k_ext != NULL) bytes (0: none needed; may then be
 *                  NULL); calls that may overlap need separate workspaces
 *   stage        : nonzero: the staging pass writes the workspace (any prior
 *                  content) before the kernel reads it.  0: no staging pass;
 *                  the workspace holds what an earlier call with stage != 0
 *                  wrote for a layer with the same source layer (a KV-shared
 *                  layer and its source stage the same slab), the same
 *                  pages, cu_q, prefix_lens, k_ext / v_ext contents,
 *                  num_seqs, max_q_len and max_kv_len, with no store to
 *                  those positions since; otherwise the results are wrong.
 *                  Ignored where nothing is staged.
 * Other arguments as in pakv_paged_attn_extend.  Errors: PAKV_ERR_WORKSPACE for
 * a missing or short workspace, else as pakv_paged_attn_extend. */
size_t pakv_extend_staging_bytes(const pakv_layer_map* map, int32_t layer, int32_t num_seqs, int32_t max_q_len,
                                 int32_t max_kv_len, int32_t packed);
pakv_status pakv_paged_attn_extend_staged(const pakv_layer_map* map, int32_t layer, const pakv_pages* pages,
                                          const int32_t* cu_q, const int32_t* prefix_lens,
                                          const void* q, const void* k_ext, const void* v_ext, void* out,
                                          int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                                          int32_t stage, void* stream);

/* ---- Decode step graphs ---------------------------------------------------------
 * A whole decode step of a layer stack, captured once per batch-size bucket
 * into a HIP graph and replayed (unsloth commit dee9371: one CUDA graph per
 * batch-size bucket; commit 749fb75: a single bucket ladder and a single pool
 * across buckets).  The step runs, on kv_lens (device int32 [max_batch], read at
 * every replay): one pakv_decode_plan per kind of layer (window, Hkv), then for
 * each step layer in order: an owning bf16 layer with k_new stores its new row
 * and decodes in one launch (pakv_paged_attn_decode_append); an owning 8-bit or
 * K=V layer with k_new runs pakv_paged_kv_store of that row at kv_lens[b] - 1,
 * then the planned decode; every other layer runs the planned decode.
 *   layers[i].q, .out          : device bf16 [max_batch][Hq][D]
 *   layers[i].k_new, .v_new    : device bf16 [max_batch][Hkv][D] (owners), or NULL
 *                                (the rows were stored before the step)
 *   pages_full, pages_sliding  : the groups' page tables (pages_sliding NULL:
 *                                pages_full for every layer)
 *   workspace                  : device memory of pakv_decode_step_workspace_bytes,
 *                                zero-filled before the first replay, shared by
 *                                every bucket; it holds the plans and one decode
 *                                workspace
 * Buffers are captured by address: they must stay allocated, and in place,
 * while the step exists.  pakv_decode_step_run(step, batch, stream) launches
 * the graph of the smallest bucket >= batch on stream (PAKV_ERR_INVALID above
 * the largest); rows batch .. bucket - 1 are decoded as well, on what the
 * caller keeps there: keep their kv_lens at 1 and their page-table rows at -1
 * (nothing is then written, and they read page 0).  Replays that may overlap
 * need separate steps and workspaces.  Creating a step captures on a stream of
 * its own and launches nothing; a call the step makes that its host-side
 * checks refuse ends the capture, and its status is returned. */
typedef struct {
    int32_t layer;
    const void* q;
    void* out;
    const void* k_new;
    const void* v_new;
} pakv_step_layer;
typedef struct pakv_decode_step pakv_decode_step;
size_t pakv_decode_step_workspace_bytes(const pakv_layer_map* map, const pakv_step_layer* layers, int32_t n_layers,
                                        int32_t max_batch, int32_t max_kv_len);
pakv_status pakv_decode_step_create(const pakv_layer_map* map, const pakv_pages* pages_full,
                                    const pakv_pages* pages_sliding, const int32_t* kv_lens, int32_t max_batch,
                                    int32_t max_kv_len, const pakv_step_layer* layers, int32_t n_layers,
                                    const int32_t* buckets, int32_t n_buckets, void* workspace,
                                    size_t workspace_bytes, pakv_decode_step** out);
pakv_status pakv_decode_step_run(pakv_decode_step* step, int32_t batch, void* stream);
/* the bucket a batch runs in, or -1 */
int32_t pakv_decode_step_bucket(const pakv_decode_step* step, int32_t batch);
void pakv_decode_step_destroy(pakv_decode_step* step);

/* ---- Page pools (host bookkeeping) -------------------------------------------
 * The two attention groups want different page lifetimes: the sliding group
 * releases pages the full group still reads (pegainfer issue #807,
 * Description, first paragraph), so each group gets its own pool and its own
 * page table (pass it as the pakv_pages of that group's calls).  A window pool
 * (window W > 0) hands a sequence's pages back once no query that can still
 * come sees them; the kernels read only pages holding visible positions (an
 * extend tile may touch one page below the window: its rows are masked, so a
 * released page, reused or poisoned, changes nothing).
 *
 * pakv_page_pool_create: num_pages physical pages for max_seqs sequences of up
 *   to max_pages_per_seq pages; window 0 for a full pool.
 * pakv_page_pool_reserve: sequence seq will next store up to position end - 1
 *   and run queries at first_query or later: it then holds every page with a
 *   position in [keep_from, end), keep_from = max(0, first_query - W + 1) (0 for
 *   a full pool), and its pages wholly below keep_from go back to the pool.  A
 *   decode step with kv_len L has first_query = L - 1, end = L; an extend chunk
 *   at P has first_query = P, end = P + n.  PAKV_ERR_WORKSPACE, changing
 *   nothing, when the pool has too few free pages.
 * pakv_page_pool_release_seq: all of a sequence's pages go back.
 * pakv_page_pool_table: host int32 [max_seqs][max_pages_per_seq], -1 where no
 *   page is held; valid until the pool is destroyed.
 * pakv_page_pool_released: the pages the last reserve / release_seq gave back
 *   (copies up to cap of them into out; returns how many there were).
 * Released pages are handed out again last-released first. */
typedef struct pakv_page_pool pakv_page_pool;
pakv_status pakv_page_pool_create(int32_t num_pages, int32_t max_seqs, int32_t max_pages_per_seq, int32_t window,
                                  pakv_page_pool** out);
void pakv_page_pool_destroy(pakv_page_pool* pool);
pakv_status pakv_page_pool_reserve(pakv_page_pool* pool, int32_t seq, int32_t first_query, int32_t end);
pakv_status pakv_page_pool_release_seq(pakv_page_pool* pool, int32_t seq);
const int32_t* pakv_page_pool_table(const pakv_page_pool* pool);
int32_t pakv_page_pool_free_pages(const pakv_page_pool* pool);
int32_t pakv_page_pool_released(const pakv_page_pool* pool, int32_t* out, int32_t cap);

/* Tokens a KV byte budget holds when the window pool keeps window_share
 * tokens for every token of the full pool (FreeToken PR #898, "End to end":
 * every printed row has a window pool of one fifth of the full pool, 0.2):
 * full_tokens = floor(budget / (full_bytes + window_share * window_bytes)),
 * window_tokens = floor(window_share * full_tokens), with the bytes per token
 * of pakv_kv_bytes_per_token (owning layers only). */
pakv_status pakv_pool_tokens(const pakv_layer_map* map, int64_t budget_bytes, double window_share,
                             int64_t* full_tokens, int64_t* window_tokens);

/* Placement check.  Launches num_workgroups (1 .. 65535) workgroups on
 * stream; workgroup i writes the id of the XCD it ran on to out[i] (device
 * int32 [num_workgroups], caller-owned).  The decode kernel merges a unit's
 * partials inside one XCD's L2 when all of the unit's workgroups share a
 * class of i mod 8, which is correct when workgroups of one class always
 * share an XCD (the dispatcher hands workgroups to the XCDs in turn); this
 * call lets a test or a deployment check that on its device.
 * PAKV_ERR_INVALID for a null out or a count out of range. */
pakv_status pakv_workgroup_xcds(int32_t* out, int32_t num_workgroups, void* stream);

/* Optional decode checks, for every decode call made while they are on (a
 * process-wide setting; 0 turns them off, the default).
 *   PAKV_CHECK_XCD_PLACEMENT: each workgroup of a unit that merges inside one
 *     XCD's L2 marks its XCD in the unit's arrival word when it starts the
 *     unit, and the merging workgroup raises PAKV_DECODE_XCD_SPLIT in the
 *     status word when more than one XCD took part.  It costs a device-scope
 *     atomic per such workgroup and unit (about 5% of the E2B-like decode
 *     step), so it is for tests and bring-up on a new device.
 * PAKV_ERR_INVALID for unknown bits. */
#define PAKV_CHECK_XCD_PLACEMENT 1
pakv_status pakv_set_decode_checks(int32_t flags);

/* Page-id bounds diagnostics.  In every build, a page-table entry outside
 * [0, num_pages) met for a position a call uses (or a position past the
 * table's width) never moves an access outside the slab: decode and extend
 * read page 0 in its place (wrong values for those keys), and a store drops
 * the row.  A build with PAKV_DEBUG_BOUNDS defined (libpakv_bounds.so, built
 * beside libpakv.so) also counts them on the device, per kind:
 *   counts[0]  entries met by decode plans (pakv_decode_plan and the calls
 *              that plan for themselves), once per chunk;
 *   counts[1]  rows dropped by pakv_paged_kv_store;
 *   counts[2]  entries met by extend calls, once per workgroup that reads
 *              the page (so a bad page may count several times).
 * The counts belong to the current device and add up over calls until
 * pakv_debug_bounds_reset.  Both calls first wait for all work on the current
 * device.  Other builds: PAKV_ERR_UNSUPPORTED (nothing is counted there). */
#define PAKV_DEBUG_COUNTS 3
pakv_status pakv_debug_bounds_counts(uint32_t counts[PAKV_DEBUG_COUNTS]);
pakv_status pakv_debug_bounds_reset(void);

/* Kernel timing hook, for benchmarks and profilers.  events points to 2 *
 * n_pairs hipEvent_t handles (caller-owned, created in the HIP runtime the
 * library runs in); while the hook is set, each store / decode / extend call
 * on the calling thread whose kernel is selected by kernel_mask records
 * events[2*i] on its stream just before that kernel's launch and
 * events[2*i + 1] just after it, for i = 0, 1, ... until the n_pairs pairs
 * are used.  events == NULL clears the hook.  The hook adds no
 * synchronisation; elapsed times are read by the caller (hipEventElapsedTime). */
#define PAKV_TIME_STORE 1           /* the store kernel */
#define PAKV_TIME_DECODE 2          /* the decode kernel */
#define PAKV_TIME_EXTEND 8          /* the extend kernel */
#define PAKV_TIME_STAGE 16          /* the staging pass of pakv_paged_attn_extend_staged */
pakv_status pakv_set_timing_events(void* const* events, int32_t n_pairs, int32_t kernel_mask);
/* Number of event pairs recorded on this thread since the hook was last set. */
int32_t pakv_timing_pairs_used(void);

#ifdef __cplusplus
}
#endif

#endif /* PAKV_H */
