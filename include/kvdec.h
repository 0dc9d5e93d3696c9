/*
 * kvdec.h -- C ABI of libkvdec.so: the single-token KV-cached decode step
 * (append the new token's K/V rows, then attend one query per head over the
 * cached rows and, for encoder-decoder models, over static encoder K/V) on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (docs.rs source pages; cited by page and item):
 *   [WA-DEC]  whisper-apr 0.3.3, src/model/decoder_generated.rs
 *   [WA-CUDA] whisper-apr 0.3.0, src/cuda/impl_generated.rs
 *   [FO-Q2]   franken_ocr 0.8.0, src/native_engine/decoder_qwen2.rs
 *   [CERA]    cera 0.5.4, src/model/whisper.rs
 *   [LAT-Q8]  lattice-inference 0.4.0, src/forward/cpu_q8.rs
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are HIP device pointers; (host) are host
 *     pointers.  All device memory (caches, lengths, q, out, workspace) is
 *     owned by the caller; the library never allocates, frees or keeps
 *     device memory, never synchronises and never creates streams.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued asynchronously on it, in call order.
 *   - Device pointers must be non-NULL and 16-byte aligned.
 *   - Return value: KVDEC_OK or a kvdec_status error code.  Every argument,
 *     shape and capacity check runs before anything is enqueued: on any
 *     error other than KVDEC_E_HIP nothing has been enqueued and no device
 *     or host state has changed.  KVDEC_E_HIP means a launch was refused by
 *     the runtime; launches the call made before it stay enqueued, and the
 *     host mirrors describe what they do (calls where that matters say so).
 *     kvdec_last_error() describes the failure (thread-local string).
 *   - head_dim is 64.  K/V elements are IEEE binary32 (KVDEC_F32) or
 *     bfloat16 bit patterns (KVDEC_BF16); q and out are always binary32.
 *   - A handle keeps a host mirror of its lengths: calls on one handle must
 *     not overlap from several host threads (distinct handles are
 *     independent), and calls that touch the same cache or workspace must be
 *     ordered on the device (one stream, or events between streams).
 */
#ifndef KVDEC_H
#define KVDEC_H

#include <stddef.h>
#include <stdint.h>

/* Every entry point is exported with default visibility; the library hides
 * everything else. */
#if defined(__GNUC__)
#define KVDEC_API __attribute__((visibility("default")))
#else
#define KVDEC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVDEC_OK = 0,
    KVDEC_E_INVALID = 1,   /* NULL / misaligned pointer, non-positive size, unknown dtype */
    KVDEC_E_SHAPE = 2,     /* head_dim != 64, heads not a multiple of KV heads, rows > capacity */
    KVDEC_E_OVERFLOW = 3,  /* an append would exceed a sequence's capacity */
    KVDEC_E_STATIC = 4,    /* append/self-attend on a static (encoder) cache, or cross on a dynamic one */
    KVDEC_E_WORKSPACE = 5, /* workspace smaller than kvdec_workspace_bytes() */
    KVDEC_E_HIP = 6        /* a HIP launch failed; see kvdec_last_error() */
} kvdec_status;

typedef enum { KVDEC_F32 = 0, KVDEC_BF16 = 1 } kvdec_dtype;

#define KVDEC_HEAD_DIM 64
#define KVDEC_ROW_ALIGN 64     /* padded capacity granule, rows */
#define KVDEC_MIN_CHUNK 64     /* smallest split-sequence chunk, rows */
#define KVDEC_MAX_CHUNK 4096   /* largest split-sequence chunk, rows */
#define KVDEC_MAX_GROUP 8      /* query heads per KV head supported */
#define KVDEC_REPLAY_AUTO (-1) /* kvdec_set_replay_mode: pick the chunk from current lengths */
#define KVDEC_MAX_FUSED_BATCH 512 /* largest batch kvdec_append_attend runs as one launch */
#define KVDEC_MAX_PAGED_FUSED_BATCH 256 /* largest batch kvdec_paged_append_attend runs as one launch */
#define KVDEC_NOALLOC_SCRATCH_BYTES 16777216 /* device scratch of kvdec_append_attend_noalloc (16 MiB per GPU) */

/* Opaque host-side handle: the cache description plus a host mirror of the
 * per-sequence lengths (used for validation and launch sizing, so no call
 * ever reads the lengths back from the device). */
typedef struct kvdec_cache kvdec_cache;

/*
 * Cache description.  Layout is head-major and padded:
 *   k, v : (device) [batch][n_kv_heads][kvdec_padded_capacity(capacity)][64]
 *          elements of `dtype`.  One row is 256 B (f32) or 128 B (bf16), so a
 *          (sequence, KV head) pair is one contiguous run of rows.
 *   lens : (device) int32[batch], rows currently held per sequence.
 * Sliding-window ring (window == capacity, dynamic caches only): lens[b]
 * counts every token the sequence has seen; token t lives in row t % window,
 * and attention reads the last min(lens[b], window) tokens -- the circular
 * buffer of [WA-DEC] `CircularKVBuffer` (slot = position mod window) and the
 * window of [WA-DEC] `StreamingKVCache`.  Appends never overflow a ring.
 * This is the head-first GPU cache of [WA-CUDA]
 * `init_gpu_decoder_kv_cache_head_first` ([n_heads, max_seq_len, head_dim] per
 * layer) extended by a batch axis and row padding; one handle is one layer's
 * self-attention cache (is_static = 0) or one layer's encoder cross-attention
 * cache (is_static = 1; [CERA] `WhisperCrossAttentionCache`, computed once per
 * audio and never appended to).
 */
typedef struct {
    int32_t batch;       /* sequences, >= 1 */
    int32_t n_kv_heads;  /* KV heads, >= 1 */
    int32_t head_dim;    /* must be 64 */
    int32_t capacity;    /* rows each sequence may hold, >= 1 */
    int32_t dtype;       /* kvdec_dtype */
    int32_t is_static;   /* 0: self cache (appendable); 1: static encoder cache */
    int32_t window;      /* 0: linear cache; == capacity: sliding-window ring (see below) */
    int32_t reserved0;   /* must be 0 */
    void* k;             /* (device) */
    void* v;             /* (device) */
    int32_t* lens;       /* (device) */
} kvdec_cache_desc;

/* Rows per (sequence, KV head) actually laid out for `capacity`: capacity
 * rounded up to a multiple of KVDEC_ROW_ALIGN.  Returns 0 for capacity < 1. */
KVDEC_API int32_t kvdec_padded_capacity(int32_t capacity);

/* Create a handle over caller-owned memory and write the initial lengths
 * lens_host[batch] (host) to desc->lens on `stream`.  Cache contents are not
 * touched.  Errors: KVDEC_E_INVALID (NULL/misaligned pointers, batch < 1,
 * unknown dtype, a static ring, reserved0 != 0), KVDEC_E_SHAPE (head_dim !=
 * 64, window not 0 or capacity, a length outside [0, capacity] for a linear
 * cache or negative for a ring).  *out receives the handle (host). */
KVDEC_API int32_t kvdec_cache_create(const kvdec_cache_desc* desc, const int32_t* lens_host,
                           void* stream, kvdec_cache** out);

/* Release the handle (host memory only; the caller's device memory is not freed). */
KVDEC_API void kvdec_cache_destroy(kvdec_cache* cache);

/* Set every sequence's length from lens_host[batch] (host), device and mirror,
 * leaving cache rows untouched ([WA-DEC] `LayerKVCache::reset` keeps the
 * storage).  Errors: KVDEC_E_INVALID, KVDEC_E_SHAPE (length outside
 * [0, capacity]). */
KVDEC_API int32_t kvdec_reset_lens(kvdec_cache* cache, const int32_t* lens_host, void* stream);

/* Copy the host mirror of the lengths into lens_out[batch] (host).  No device
 * access.  Errors: KVDEC_E_INVALID (also while the mirror is unknown after
 * leaving replay mode; see kvdec_set_replay_mode). */
KVDEC_API int32_t kvdec_get_lens(const kvdec_cache* cache, int32_t* lens_out);

/*
 * Seed rows [0, rows) of every sequence from token-major data and set every
 * length to `rows`: the interleaved-to-head-first permute [L, H*64] ->
 * [H, L, 64] of [WA-CUDA] `populate_cross_kv_caches_gpu` (encoder K/V), also
 * usable for a prefill of the self cache ([FO-Q2] `Qwen2KvCache::seed`).
 *   k_tok, v_tok : (device) [batch][rows][n_kv_heads*64] elements of dtype.
 * Allowed on static and dynamic caches.  Errors: KVDEC_E_INVALID,
 * KVDEC_E_SHAPE (rows < 0 or rows > capacity).
 */
KVDEC_API int32_t kvdec_seed(kvdec_cache* cache, const void* k_tok, const void* v_tok, int32_t rows,
                   void* stream);

/*
 * Append one token: for every sequence b and KV head g, copy k_new[b][g][:]
 * and v_new[b][g][:] into row lens[b] of the cache, then lens[b] += 1.
 *   k_new, v_new : (device) [batch][n_kv_heads][64] elements of the cache dtype.
 * A pure byte copy (bit-exact, no conversion): [WA-DEC]
 * `LayerKVCache::append`, [FO-Q2] `Qwen2KvCache::append`, and the head-first
 * scatter at row `pos` of [WA-CUDA] `kv_cache_scatter_gpu`.
 * Errors: KVDEC_E_OVERFLOW when any lens[b] + 1 > capacity -- checked before
 * anything is enqueued, like the "cache overflow" check of
 * `LayerKVCache::append`; KVDEC_E_STATIC on a static cache; KVDEC_E_INVALID.
 */
KVDEC_API int32_t kvdec_append(kvdec_cache* cache, const void* k_new, const void* v_new, void* stream);

/*
 * Append with a sliding window that keeps an overlap: the streaming cache of
 * [WA-DEC] `StreamingKVCache` (`append_with_slide`, `slide_window`) on a
 * linear cache whose capacity is the window.  For every sequence b whose new
 * row would pass the capacity (lens[b] + 1 > capacity), the cache first
 * keeps only its last keep = min(overlap, capacity / 2) rows -- rows
 * lens[b] - keep .. lens[b] - 1 move to rows 0 .. keep - 1 (the page caps
 * the overlap at half the window) -- and lens[b] becomes keep; then the row
 * is appended as kvdec_append does.  Other sequences append normally.
 * Attention then reads the kept rows and the new one.  The decision is
 * taken on the device from the device lengths (so the call is capturable
 * in replay mode too), and mirrored on the host.
 *   k_new, v_new : as kvdec_append
 *   overlap      : rows to keep when a sequence slides, >= 0
 *   slid_out     : (host) NULL, or int32[batch]: 1 where the sequence slid, else
 *                  0 (from the host mirror)
 * Errors: KVDEC_E_STATIC (static cache), KVDEC_E_INVALID (a ring cache,
 * overlap < 0, pointers, unknown lengths after replay mode).
 */
KVDEC_API int32_t kvdec_append_slide(kvdec_cache* cache, const void* k_new, const void* v_new,
                                     int32_t overlap, int32_t* slid_out, void* stream);

/*
 * Append with rotary position embedding: like kvdec_append, but k_new holds
 * the un-rotated keys; each is rotated at its token's position (the
 * sequence's length before this append) before it is stored, and, when q is
 * given, the queries are rotated at the same position into q_rot -- the
 * order of [FO-Q2] `qwen2_decode_step` (RoPE on q and k, then append, then
 * attend).  NEOX rotate-half: dims (i, i+32) rotate by pos * theta^(-2i/64)
 * ([LAT-Q8] `full_attention_step_q8` stride-half pairing; theta = 1e6 for
 * Qwen2 per [FO-Q2]).  Angles and rotation in double, rounded to float (and
 * to bf16, nearest even, for bf16 caches).  V rows are copied unchanged.
 *   q, q_rot : (device) float [batch][n_q_heads][64], both NULL or both
 *              given; they may be the same buffer.
 * Errors: those of kvdec_append, plus KVDEC_E_INVALID (theta not a positive
 * finite number, only one of q / q_rot given) and KVDEC_E_SHAPE (n_q_heads
 * not a positive multiple of n_kv_heads).
 */
KVDEC_API int32_t kvdec_append_rope(kvdec_cache* cache, const void* k_new, const void* v_new, float theta,
                          const float* q, float* q_rot, int32_t n_q_heads, void* stream);

/* Workspace bytes any attend call on `cache` with n_q_heads query heads may
 * need (split-sequence partial results).  Its contents need no
 * initialisation and carry nothing between calls; calls sharing one
 * workspace must not run concurrently (use one stream, or one workspace per
 * stream).  0 on invalid arguments. */
KVDEC_API size_t kvdec_workspace_bytes(const kvdec_cache* cache, int32_t n_q_heads);

/*
 * Decode attention of one query per head over the cached rows of each
 * sequence (self-attention; the cache must be dynamic):
 *   out[b][h][:] = sum_j softmax_j(scale * q[b][h] . K[b][g][j]) * V[b][g][j][:]
 * for j < lens[b], g = h / (n_q_heads / n_kv_heads).
 *   q   : (device) float [batch][n_q_heads][64]
 *   out : (device) float [batch][n_q_heads][64]
 *   ws  : (device) workspace of ws_bytes >= kvdec_workspace_bytes(cache, n_q_heads)
 * Semantics follow [FO-Q2] `decode_attn_head` / `qwen2_decode_attention`
 * (every cached row attended, no mask: causality is implicit because the
 * cache holds only positions <= the current one, the current one included
 * after kvdec_append), [LAT-Q8] `full_attention_step_q8` (GQA mapping
 * kvh = qh / groups; a softmax denominator that is not > 0, e.g. from a NaN
 * score, yields a zero output row) and [CERA] `multi_head_attention`.
 * A sequence with length 0 yields a zero row.  scale is usually 1/sqrt(64).
 * chunk_rows: rows per split-sequence chunk; 0 picks automatically, else a
 * multiple of 64 in [KVDEC_MIN_CHUNK, KVDEC_MAX_CHUNK].  For a given
 * chunk_rows the result for a sequence is bitwise independent of the other
 * sequences in the batch (and of the batch size), and bitwise the same
 * through kvdec_attend_self, kvdec_append_attend and
 * kvdec_append_attend_at; the one exception is replay mode without a
 * horizon, whose capacity-sized grids may split a chunk's rows over waves
 * differently from other launches (results within the tolerance, not
 * bitwise equal to them).  One kernel launch per call, plus a log-sum-exp
 * merge launch when some sequence spans more than one chunk.
 * Errors: KVDEC_E_SHAPE (n_q_heads not a positive multiple of n_kv_heads, or
 * group > KVDEC_MAX_GROUP), KVDEC_E_STATIC, KVDEC_E_WORKSPACE, KVDEC_E_INVALID,
 * KVDEC_E_HIP.
 */
KVDEC_API int32_t kvdec_attend_self(const kvdec_cache* cache, const float* q, int32_t n_q_heads,
                          float scale, int32_t chunk_rows, float* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * kvdec_append followed by kvdec_attend_self, as one call: the decode step
 * of one layer's self-attention.  Same arguments and errors as the two
 * calls (everything is checked before anything is enqueued); results, cache
 * bytes and lengths are bitwise those of the two calls.  The append is fused
 * into the attend launch -- the append-plus-attend cached call of [WA-CUDA]
 * `flash_attention_cached`: each workgroup reads the rows it attends, and the
 * one whose chunk holds the new slot first stores the new K/V row there.
 *   - batch <= KVDEC_MAX_FUSED_BATCH outside replay mode: one launch (plus
 *     the merge launch when a sequence spans several chunks); the pre-append
 *     lengths go by value from the host mirror and the launch bumps them.
 *   - otherwise (replay mode, larger batches): the attend launch reads the
 *     lengths from the device and the merge launch, which then always runs,
 *     bumps them; two launches, capturable in a graph like every call in
 *     replay mode.  As with kvdec_append in replay mode, a full linear
 *     cache keeps its length and gets no row.
 */
KVDEC_API int32_t kvdec_append_attend(kvdec_cache* cache, const void* k_new, const void* v_new,
                                      const float* q, int32_t n_q_heads, float scale,
                                      int32_t chunk_rows, float* out, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * One decoder layer's whole attention step for an encoder-decoder model:
 * kvdec_append_attend (or kvdec_append_attend_at) on the self cache, then
 * kvdec_attend_cross on the static encoder cache, as one call -- the
 * self-then-cross order of one
 * decoder block in [CERA] `decode_step_into` and [WA-CUDA]
 * `forward_decoder_block_gpu_stream`.  Both parts run in one attend launch
 * (plus one log-sum-exp merge launch when a sequence of either part spans
 * several chunks): the cross part's workgroups come first in the grid, the
 * self part's, with the append fused in, after them.  Outputs, cache bytes
 * and lengths are bitwise those of the two calls made with the chunk sizes
 * the call used: chunk_self and chunk_cross where given, else each call's
 * own automatic choice -- except that where the two parts would then run on
 * workgroups of different shapes (f32 with 1-2 query heads per KV head, one
 * chunk size >= 256 rows and the other smaller), an automatic part takes
 * 192-row chunks so that both share the launch.  If both sizes were given
 * and still differ in shape, the call makes the two calls instead.
 *   self_cache  : dynamic cache, appended to (KVDEC_E_STATIC otherwise)
 *   cross_cache : static cache of the same batch, n_kv_heads and dtype
 *                 (KVDEC_E_STATIC if dynamic, KVDEC_E_SHAPE if they differ)
 *   lens_host   : (host) NULL, or int32[batch] positions: the self part is
 *                 then kvdec_append_attend_at(lens_host) instead (the step
 *                 at explicit positions, a rewind included, with no launch
 *                 of its own where the step is one launch)
 *   k_new, v_new, q_self, out_self : as kvdec_append_attend
 *   q_cross, out_cross             : as kvdec_attend_cross (same n_q_heads)
 *   ws : (device) workspace of ws_bytes >= kvdec_workspace_bytes(self_cache,
 *        n_q_heads) + kvdec_workspace_bytes(cross_cache, n_q_heads)
 * Every check of both calls runs before anything is enqueued.  Errors:
 * those of the two calls.
 */
KVDEC_API int32_t kvdec_append_attend_cross(kvdec_cache* self_cache, const kvdec_cache* cross_cache,
                                            const int32_t* lens_host, const void* k_new,
                                            const void* v_new,
                                            const float* q_self, const float* q_cross,
                                            int32_t n_q_heads, float scale, int32_t chunk_self,
                                            int32_t chunk_cross, float* out_self, float* out_cross,
                                            void* ws, size_t ws_bytes, void* stream);

/*
 * kvdec_append_attend for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same step, the same kernels and bitwise the
 * same results, cache bytes and lengths, with the split-sequence partials
 * held in the library's own device scratch instead of a workspace
 * argument.  The call allocates and frees nothing.  The scratch is a
 * static array of KVDEC_NOALLOC_SCRATCH_BYTES on each GPU the library runs
 * on (held until the process ends); its address is looked up once per GPU,
 * on the first call made with that GPU current.  A call needs
 * 264 * n_q_heads * C + 4 * batch bytes of it (each part rounded up to 256
 * bytes), where C is the number of chunks of the launch: the sum over
 * sequences of max(1, ceil(rows / chunk_rows)) with rows = lens[b] + 1 (the
 * window of a ring at most), or, in replay mode, the rows a sequence can
 * reach (the capacity or the horizon).  Larger calls fail with
 * KVDEC_E_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares its scratch, and the scratch keeps only what the last call left:
 * calls whose launches overlap on one GPU (other streams, other threads,
 * other handles) race and must be ordered by the caller.  Arguments and
 * other errors as kvdec_append_attend without ws / ws_bytes; KVDEC_E_HIP
 * also when the scratch address cannot be found.
 */
KVDEC_API int32_t kvdec_append_attend_noalloc(kvdec_cache* cache, const void* k_new,
                                              const void* v_new, const float* q,
                                              int32_t n_q_heads, float scale, int32_t chunk_rows,
                                              float* out, void* stream);

/*
 * kvdec_reset_lens(lens_host) then kvdec_append_attend, as one call: the
 * decode step at explicit positions ([CERA] `decode_step_into` takes the
 * token's position and leaves the cache length at position + 1), which also
 * rewinds a sequence, for example after draft tokens were rejected.
 * lens_host[b] (host) is the number of tokens sequence b keeps before this
 * one; afterwards it holds lens_host[b] + 1.  Where
 * kvdec_append_attend is one launch, the positions go to it by value and it
 * writes the device lengths, so the rewind costs no launch of its own;
 * otherwise the lengths are set on the device first (a launch of its own),
 * and if the attend launch is then refused (KVDEC_E_HIP) the lengths stay
 * set to lens_host, on the device and in the host mirror alike, as after
 * kvdec_reset_lens.  Errors: those of the two calls (a linear cache needs
 * lens_host[b] < capacity).
 */
KVDEC_API int32_t kvdec_append_attend_at(kvdec_cache* cache, const int32_t* lens_host,
                                         const void* k_new, const void* v_new, const float* q,
                                         int32_t n_q_heads, float scale, int32_t chunk_rows,
                                         float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Cross-attention over a static encoder cache: the same computation as
 * kvdec_attend_self over every seeded row (1500 for Whisper's 30 s window),
 * with the decoder's cross query: [CERA] `decode_step_into` cross block and
 * [WA-CUDA] `forward_decoder_block_gpu_stream` (incremental attention with
 * seq_len = encoder length).  The cache must be static (KVDEC_E_STATIC otherwise).
 */
KVDEC_API int32_t kvdec_attend_cross(const kvdec_cache* cache, const float* q, int32_t n_q_heads,
                           float scale, int32_t chunk_rows, float* out, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Paged KV cache: K and V live in a pool of fixed-size pages shared by all
 * sequences, and each sequence owns a block table of page ids -- the paged
 * cache of [WA-DEC] `PagedDecoderKVCache` over realizar's `PagedKvCache`
 * (page = position / page size, offset = position % page size; on an
 * allocation failure nothing changes).  The library keeps the page
 * allocator (a host-side free list) and host mirrors of the lengths and
 * block tables; the caller owns every device buffer.
 *   k_pages, v_pages : (device) [n_kv_heads][num_pages][page_rows][64] elements
 *                      of dtype, head-major: one page id covers every KV head,
 *                      one (KV head, page) is a contiguous run of rows, and
 *                      consecutive pages of one head are adjacent
 *   block_table      : (device) int32 [batch][max_pages_per_seq]; written by
 *                      the library only: -1 after create, page ids as pages
 *                      are taken; read for the rows a sequence holds and, in
 *                      replay mode, for the row an append stores (then every
 *                      entry past a sequence's pages is -1)
 *   lens             : (device) int32 [batch], all zero after create
 * ------------------------------------------------------------------------- */
typedef struct kvdec_paged kvdec_paged;

typedef struct {
    int32_t batch;              /* sequences, >= 1 */
    int32_t n_kv_heads;         /* >= 1 */
    int32_t head_dim;           /* must be 64 */
    int32_t dtype;              /* kvdec_dtype */
    int32_t page_rows;          /* rows per page: a power of two in [16, 4096] */
    int32_t num_pages;          /* pages in the pool, >= 1 */
    int32_t max_pages_per_seq;  /* block table width, >= 1 */
    int32_t reserved0;          /* must be 0 */
    void* k_pages;
    void* v_pages;
    int32_t* block_table;
    int32_t* lens;
} kvdec_paged_desc;

/* Create a paged cache: every sequence empty, every page free; writes zero
 * lengths and a block table of -1 on `stream`.  Errors: KVDEC_E_INVALID,
 * KVDEC_E_SHAPE (head_dim, page_rows not a power of two in range, block
 * table or rows per sequence too large for int32 indices). */
KVDEC_API int32_t kvdec_paged_create(const kvdec_paged_desc* desc, void* stream, kvdec_paged** out);
KVDEC_API void kvdec_paged_destroy(kvdec_paged* paged);

/* Append one token to every sequence (same k_new / v_new layout as
 * kvdec_append).  A sequence whose new row starts a page takes a free page
 * (lowest-numbered first, in sequence order).  Errors: KVDEC_E_OVERFLOW
 * when a sequence would exceed max_pages_per_seq * page_rows or the pool
 * has too few free pages -- checked before anything changes; a failed
 * launch (KVDEC_E_HIP) returns the pages taken. */
KVDEC_API int32_t kvdec_paged_append(kvdec_paged* paged, const void* k_new, const void* v_new, void* stream);

/* End sequence `seq`: its pages return to the pool and its length becomes 0
 * (written on `stream`; in replay mode its block table entries become -1). */
KVDEC_API int32_t kvdec_paged_release(kvdec_paged* paged, int32_t seq, void* stream);

/* Give the empty sequence `seq` ceil(len / page_rows) free pages and the
 * length `len` (table entries and length written on `stream`): the hand-off
 * from a prefill that writes the rows into those pages itself (read their
 * ids with kvdec_paged_get_table).  Errors: KVDEC_E_INVALID (bad seq, or
 * the sequence is not empty), KVDEC_E_OVERFLOW (len beyond the block table,
 * or too few free pages; nothing changes). */
KVDEC_API int32_t kvdec_paged_reserve(kvdec_paged* paged, int32_t seq, int32_t len, void* stream);

/* Shorten sequences to lens_host[batch] (each <= its current length; after
 * replay mode, each <= the rows its pages hold): pages past the new ends
 * return to the pool (in replay mode their block table entries become -1),
 * rows before them are kept --
 * rolling back speculative tokens, replaying a benchmark cycle, or setting
 * the lengths after replay mode.  Errors: KVDEC_E_INVALID, KVDEC_E_SHAPE (a
 * length outside that range). */
KVDEC_API int32_t kvdec_paged_truncate(kvdec_paged* paged, const int32_t* lens_host, void* stream);

/* Host mirrors: lengths [batch], block table [batch][max_pages_per_seq]
 * (-1 where no page is held), and the number of free pages (-1 for NULL). */
KVDEC_API int32_t kvdec_paged_get_lens(const kvdec_paged* paged, int32_t* lens_out);
KVDEC_API int32_t kvdec_paged_get_table(const kvdec_paged* paged, int32_t* table_out);
KVDEC_API int32_t kvdec_paged_free_pages(const kvdec_paged* paged);

/* Workspace for kvdec_paged_attend (same rules as kvdec_workspace_bytes). */
KVDEC_API size_t kvdec_paged_workspace_bytes(const kvdec_paged* paged, int32_t n_q_heads);

/* Decode attention over the paged cache: the computation of
 * kvdec_attend_self, with each row found through the block table. */
KVDEC_API int32_t kvdec_paged_attend(const kvdec_paged* paged, const float* q, int32_t n_q_heads,
                           float scale, int32_t chunk_rows, float* out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * kvdec_paged_append then kvdec_paged_attend, as one call (the one-launch
 * decode step of kvdec_append_attend for the paged layout): pages are taken
 * exactly as kvdec_paged_append takes them, and output, pool rows, block
 * table and lengths are bitwise those of the two calls.  Up to
 * KVDEC_MAX_PAGED_FUSED_BATCH sequences run as one attend launch (plus the
 * merge when a sequence spans several chunks): the pre-append lengths and
 * each sequence's fresh page (if its new row starts one) go to the kernel by
 * value, the workgroup holding the new row's slot stores it, and head 0's
 * workgroup gives the block table the fresh page and bumps the length.
 * Larger batches run the two calls.  Arguments as kvdec_paged_append and
 * kvdec_paged_attend; every check runs before anything changes.  Errors:
 * theirs (KVDEC_E_INVALID, KVDEC_E_SHAPE, KVDEC_E_OVERFLOW,
 * KVDEC_E_WORKSPACE, KVDEC_E_HIP; a failed launch returns the pages taken).
 */
KVDEC_API int32_t kvdec_paged_append_attend(kvdec_paged* paged, const void* k_new, const void* v_new,
                                            const float* q, int32_t n_q_heads, float scale,
                                            int32_t chunk_rows, float* out, void* ws, size_t ws_bytes,
                                            void* stream);

/*
 * Replay mode for a paged cache: the paged decode step captured once in a
 * HIP graph and replayed for consecutive tokens, as kvdec_set_replay_mode
 * does for a contiguous cache ([WA-CUDA] `forward_decoder_token_gpu_stream`
 * over the paged cache of [WA-DEC] `PagedDecoderKVCache`).  chunk_rows as
 * for kvdec_set_replay_mode (> 0, KVDEC_REPLAY_AUTO, or 0 to leave).  In
 * replay mode kvdec_paged_attend is launched for max_pages_per_seq *
 * page_rows rows (or per sequence, kvdec_paged_set_replay_horizon) with the
 * merge launch always made, kvdec_paged_append and
 * kvdec_paged_append_attend read the lengths from the device (the latter as
 * one attend launch that stores the new rows, plus the merge launch, which
 * bumps the lengths), and an append takes no page: every row's page must
 * already be in the block table, put there by kvdec_paged_prepare (outside
 * the graph) before the replays that append it.  An append whose row has no
 * page leaves that sequence's row and length unchanged (and
 * kvdec_paged_append_attend then attends the rows the sequence had).
 * Entering replay mode sets -1 on `stream` in every block table entry past a
 * sequence's pages, and in replay mode pages returned to the pool
 * (kvdec_paged_release, kvdec_paged_truncate) get -1 there too, so such a
 * row never lands in another sequence's page.  The host mirror counts the prepared rows, which
 * the replays may not all have appended, so leaving replay mode (0) makes
 * calls that need the exact lengths (kvdec_paged_append, kvdec_paged_attend,
 * kvdec_paged_append_attend, kvdec_paged_reserve, kvdec_paged_get_lens,
 * entering replay mode again) fail with KVDEC_E_INVALID until
 * kvdec_paged_truncate sets the lengths.
 * Errors: KVDEC_E_INVALID (chunk_rows, or entering with unknown lengths),
 * KVDEC_E_HIP.
 */
KVDEC_API int32_t kvdec_paged_set_replay_mode(kvdec_paged* paged, int32_t chunk_rows, void* stream);

/* kvdec_set_replay_horizon for a paged cache: replay grids cover each
 * sequence's mirrored rows (in replay mode, the rows prepared so far) plus
 * `tokens`, capped at max_pages_per_seq * page_rows, with NaN output rows
 * for a sequence a replay has outgrown; 0 sizes for that cap.  Errors:
 * KVDEC_E_INVALID (tokens < 0). */
KVDEC_API int32_t kvdec_paged_set_replay_horizon(kvdec_paged* paged, int32_t tokens);

/* In replay mode: give every sequence the pages for its next n_tokens rows
 * (from the pool, in sequence order, lowest-numbered first, as
 * kvdec_paged_append takes them), write them to the device block table on
 * `stream`, and advance the host mirror by n_tokens per sequence -- the
 * appends the next replays make.  Not capturable (it picks pages on the
 * host); call it between replays.  Errors: KVDEC_E_INVALID (not in replay
 * mode, n_tokens < 0), KVDEC_E_OVERFLOW (a sequence would exceed
 * max_pages_per_seq * page_rows rows, or too few free pages; nothing
 * changes), KVDEC_E_HIP (the pages are returned). */
KVDEC_API int32_t kvdec_paged_prepare(kvdec_paged* paged, int32_t n_tokens, void* stream);

/*
 * Replay mode, for decode steps captured once in a HIP graph and replayed
 * for consecutive tokens (the graph-replayed decoder step of [WA-CUDA]
 * `forward_decoder_token_gpu_stream`: one stream, no host synchronisation).
 * chunk_rows > 0 (a multiple of 64 in [KVDEC_MIN_CHUNK, KVDEC_MAX_CHUNK])
 * enters replay mode with that fixed chunk size, KVDEC_REPLAY_AUTO with the
 * automatic choice for the current lengths; 0 leaves it.  In replay
 * mode every attend call is launched for the most rows a sequence can hold
 * (capacity, or the window of a ring) and the merge launch is always made
 * when a sequence can span several chunks, so the launches read the current
 * lengths from the device and stay valid as appends inside replays grow
 * them.  The host mirror of the lengths is not advanced by replays, so
 * kvdec_append does not check capacity on the host in replay mode; on the
 * device an append to a full linear cache writes nothing and leaves the
 * length unchanged (a ring never fills).  kvdec_reset_lens keeps working and
 * is capturable.  Leaving replay mode (0) on a dynamic cache forgets the host
 * mirror, since replays may have appended: until kvdec_reset_lens,
 * kvdec_seed or kvdec_append_attend_at sets the lengths again, calls that
 * size launches or check capacity from the mirror (kvdec_append,
 * kvdec_append_rope, kvdec_attend_self, kvdec_append_attend) and
 * kvdec_get_lens fail with KVDEC_E_INVALID.  Errors: KVDEC_E_INVALID.
 */
KVDEC_API int32_t kvdec_set_replay_mode(kvdec_cache* cache, int32_t chunk_rows);

/* Replay grids sized per sequence instead of for the capacity: with
 * tokens > 0, every attend launch made in replay mode covers, for each
 * sequence, the rows the host mirror holds at the call plus `tokens` more
 * (capped at the capacity or window) -- enough for a captured step replayed
 * for `tokens` appends from the lengths at capture, with fewer surplus
 * workgroups than a capacity-sized grid.  The mirror is what the calls made
 * it (kvdec_reset_lens, kvdec_append_attend_at, or the appends made while
 * capturing), not what replays did on the device.  A replay whose lengths
 * have outgrown the grid writes NaN into the output rows of every sequence
 * the grid no longer covers (and a fused append leaves their lengths as they
 * are); re-capture, or reset the lengths, before that.  0 (the default)
 * sizes for the capacity.  Errors: KVDEC_E_INVALID (tokens < 0). */
KVDEC_API int32_t kvdec_set_replay_horizon(kvdec_cache* cache, int32_t tokens);

/* Static description of a status code. */
KVDEC_API const char* kvdec_status_str(int32_t status);

/* Detail of the last error raised on the calling thread ("" if none). */
KVDEC_API const char* kvdec_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVDEC_H */
