// Host side of libkvdec.so: argument validation, the host mirror of the
// per-sequence lengths, chunk-size choice and workspace sizing.  Every check
// runs before anything is enqueued, so an error leaves device and host state
// unchanged.  No device memory is allocated and no call synchronises.
#include "../../include/kvdec.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "kvdec_internal.h"

struct kvdec_paged {
    kvdec_paged_desc d;
    int32_t pshift;
    std::vector<int32_t> lens;        // host mirror of d.lens
    std::vector<int32_t> table;       // host mirror of d.block_table, -1: no page
    std::vector<int32_t> free_pages;  // pool pages not held by any sequence (a stack)
    int32_t replay_chunk = 0;         // > 0: replay mode with this fixed chunk size
    int32_t replay_horizon = 0;       // > 0: replay grids sized for the lengths + this many appends
    // In replay mode `lens` counts the rows given pages by kvdec_paged_prepare
    // (an upper bound of the device lengths).  false after replay mode was
    // left: calls that need the exact lengths fail until kvdec_paged_truncate
    // sets them.
    bool lens_known = true;
};

struct kvdec_cache {
    kvdec_cache_desc d;
    int32_t cap_pad;
    std::vector<int32_t> lens;   // host mirror of d.lens
    int32_t replay_chunk = 0;    // > 0: replay mode with this fixed chunk size
    int32_t replay_horizon = 0;  // > 0: replay grids sized for the lengths + this many appends
    // false after replay mode was left on a dynamic cache: replays may have
    // advanced the device lengths, so the mirror is not used until the
    // caller sets the lengths again (kvdec_reset_lens, kvdec_seed,
    // kvdec_append_attend_at)
    bool lens_known = true;
};

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t esz_of(int32_t dtype) { return dtype == KVDEC_F32 ? 4 : 2; }

int32_t hip_fail(hipError_t e, const char* what)
{
    return fail(KVDEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Lengths count the tokens a sequence holds.  A linear cache holds at most
// `capacity`; a sliding-window ring counts every token it has seen (it keeps
// the last `window` of them), so any non-negative length is valid.
int32_t check_lens(const int32_t* lens_host, int32_t batch, int32_t capacity, int32_t window)
{
    if (!lens_host) return fail(KVDEC_E_INVALID, "lens_host is NULL");
    for (int32_t b = 0; b < batch; ++b)
        if (lens_host[b] < 0 || (window == 0 && lens_host[b] > capacity))
            return fail(KVDEC_E_SHAPE, "length %d of sequence %d outside [0, %d]", lens_host[b], b,
                        capacity);
    return KVDEC_OK;
}

// Rows an attend call reads per sequence: min(len, window) for a ring.
std::vector<int32_t> attended_rows(const kvdec_cache* c)
{
    std::vector<int32_t> r(c->lens);
    if (c->d.window > 0)
        for (auto& x : r) x = x < c->d.window ? x : c->d.window;
    return r;
}

int64_t chunks_for(const std::vector<int32_t>& lens, int32_t T)
{
    int64_t n = 0;
    for (int32_t l : lens) {
        const int64_t c = (static_cast<int64_t>(l) + T - 1) / T;
        n += c > 0 ? c : 1;
    }
    return n;
}

// Automatic chunk size (rows per workgroup), from sweeps on MI355X, in
// terms of R = attend workgroups resident at once on the device:
//  - one chunk per sequence when the (sequence, KV head) pairs alone give at
//    least R/2 workgroups and lengths are within 2x of their mean: even work
//    per workgroup and no merge launch;
//  - otherwise chunks of about 128 KB of K and V rows (256 f32 / 512 bf16
//    rows), halved while the grid would have fewer than R/4 workgroups.
//    Sweeps over 64..2048 rows put the fastest chunk at ~128 KB for ragged
//    and for equal lengths alike (qwen2-0.5b f32: 256 rows; gqa bf16: 512;
//    whisper-base cross f32: 256); smaller chunks pay per-workgroup set-up
//    and merge work, larger ones balance ragged lengths worse.  Short
//    sequences need the R/4 floor (whisper-base self: 64 rows).
constexpr int32_t kChunkBytes = 128 * 1024;

// Whether a grid of P chunks (per KV head) can run on the CU-balanced
// placement of the MFMA kernel (plan_placement): the CUs split evenly into
// one class per KV head, at least two chunks per class, at most kMaxPlaced
// positions, and the whole grid resident at once.
bool placeable(int64_t P, int32_t n_kv_heads, int64_t resident)
{
    const int cus = kvdec::device_cus();
    if (cus <= 0 || n_kv_heads <= 0 || cus % n_kv_heads != 0) return false;
    const int64_t classes = cus / n_kv_heads;
    const int64_t per = (P + classes - 1) / classes;
    const int64_t npos = per * classes;
    return per >= 2 && npos <= kvdec::kMaxPlaced && npos * n_kv_heads <= resident;
}

int32_t auto_chunk(const std::vector<int32_t>& lens, int32_t n_kv_heads, int32_t esz,
                   int64_t resident, int32_t group = 1, bool paged = false)
{
    if (resident <= 0) resident = 2048;
    int64_t total = 0;
    int32_t longest = 0;
    bool equal = true;
    for (int32_t l : lens) {
        total += l;
        longest = l > longest ? l : longest;
        equal = equal && l == lens[0];
    }
    const int64_t pairs = static_cast<int64_t>(lens.size()) * n_kv_heads;
    if (2 * pairs >= resident && longest <= KVDEC_MAX_CHUNK &&
        static_cast<int64_t>(longest) * static_cast<int64_t>(lens.size()) <= 2 * total) {
        int32_t T = KVDEC_MIN_CHUNK;
        while (T < longest) T <<= 1;
        return T;
    }
    int32_t T = kChunkBytes / (2 * KVDEC_HEAD_DIM * esz);
    const int64_t min_blocks = resident / 4;
    while (T > KVDEC_MIN_CHUNK && chunks_for(lens, T) * n_kv_heads < min_blocks) T >>= 1;
    // Grids the MFMA kernel runs placed (bf16, grouped query heads, ragged
    // lengths, contiguous cache): the smallest chunk, in steps of 64 rows
    // down to half the size above, whose grid still fits one placed
    // residency round; the finer split balances the rows per CU better
    // (gqa, 64 sequences of 16..8192 rows: 19.75 us per step at 448 rows
    // against 20.05 at 512; at 384 the grid needs a second round and takes
    // 22.5).  Through a page pool the same split was slower (16-row pages:
    // 20.7 against 20.1 us), so paged grids keep the size above.
    if (esz == 2 && group >= 2 && !equal && !paged &&
        placeable(chunks_for(lens, T), n_kv_heads, resident)) {
        const int32_t floor_rows = T / 2 > KVDEC_MIN_CHUNK ? T / 2 : KVDEC_MIN_CHUNK;
        while (T - 64 >= floor_rows && placeable(chunks_for(lens, T - 64), n_kv_heads, resident))
            T -= 64;
    }
    return T;
}

int64_t max_chunks(const kvdec_cache* c)
{
    return static_cast<int64_t>(c->d.batch) * ((c->cap_pad + KVDEC_MIN_CHUNK - 1) / KVDEC_MIN_CHUNK);
}

// What an attend call needs to know about the cache it reads, for both the
// contiguous and the paged layouts.
struct AttendView {
    int32_t batch, n_kv_heads, dtype, cap_pad, row_limit, replay_chunk;
    int32_t replay_horizon = 0;    // replay grids: rows + horizon per sequence, else the capacity
    const void* k;
    const void* v;
    const int32_t* lens_dev;
    std::vector<int32_t> rows;     // rows attended per sequence (host mirror)
    int64_t max_chunks;            // workspace sizing bound
    const int32_t* table = nullptr;
    int32_t table_stride = 0, pshift = 0, num_pages = 0;
    const int32_t* fresh_pages = nullptr;  // paged fused append: page of a row that starts one
    // append fused into the attend launch
    const int32_t* fused_lens = nullptr;   // pre-append lengths (host mirror)
    bool fused_device = false;             // append fused, lengths from the device
    const void* k_new = nullptr;
    const void* v_new = nullptr;
    int32_t* lens_out = nullptr;
    int32_t window = 0;
    // the partials go to the library's device scratch, laid out for this
    // launch's chunks, instead of the caller's workspace (ws is ignored)
    bool use_scratch = false;
};

// Argument checks of an attend call; nothing is enqueued.
int32_t check_attend(const AttendView& v, const float* q, int32_t n_q_heads, float scale,
                     int32_t chunk_rows, const float* out, const void* ws, size_t ws_bytes)
{
    if (!aligned16(q) || !aligned16(out))
        return fail(KVDEC_E_INVALID, "q and out must be non-NULL, 16-byte aligned device pointers");
    if (n_q_heads <= 0 || n_q_heads % v.n_kv_heads != 0)
        return fail(KVDEC_E_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                    n_q_heads, v.n_kv_heads);
    const int32_t group = n_q_heads / v.n_kv_heads;
    if (group > KVDEC_MAX_GROUP)
        return fail(KVDEC_E_SHAPE, "group size %d exceeds %d", group, KVDEC_MAX_GROUP);
    if (!std::isfinite(scale)) return fail(KVDEC_E_INVALID, "scale must be finite");
    if (chunk_rows != 0 && (chunk_rows < KVDEC_MIN_CHUNK || chunk_rows > KVDEC_MAX_CHUNK ||
                            chunk_rows % 64 != 0))
        return fail(KVDEC_E_INVALID, "chunk_rows %d must be 0 or a multiple of 64 in [%d, %d]",
                    chunk_rows, KVDEC_MIN_CHUNK, KVDEC_MAX_CHUNK);
    if (v.use_scratch) return KVDEC_OK;     // sized per launch in attend_view
    const kvdec::PartialLayout part = kvdec::partial_layout(v.max_chunks, n_q_heads, v.batch);
    if (!aligned16(ws) || ws_bytes < part.bytes)
        return fail(KVDEC_E_WORKSPACE, "workspace needs %zu bytes at a 16-byte aligned address, got %zu",
                    part.bytes, ws_bytes);
    return KVDEC_OK;
}

// The chunk plan of an attend launch over view v: chunk size, grid size
// along x, whether a merge launch follows, and whether every sequence has
// exactly one chunk.
void plan_chunks(const AttendView& v, int32_t group, int32_t chunk_rows, kvdec::AttendArgs& a)
{
    a.lens = v.lens_dev;
    a.batch = v.batch;
    a.n_kv_heads = v.n_kv_heads;
    a.group = group;
    a.cap_pad = v.cap_pad;
    a.row_limit = v.row_limit;
    if (v.replay_chunk > 0) {
        // Replay mode: sized for the most rows any sequence can hold, so the
        // launch stays valid while the device lengths grow between graph
        // replays (surplus workgroups exit at once; the merge checks every
        // sequence's chunk count on the device).
        a.chunk_rows = chunk_rows ? chunk_rows : v.replay_chunk;
        const int64_t per_seq = (static_cast<int64_t>(a.row_limit) + a.chunk_rows - 1) / a.chunk_rows;
        a.n_chunks = static_cast<int64_t>(v.batch) * (per_seq > 0 ? per_seq : 1);
        a.need_merge = per_seq > 1;
        a.replay = v.replay_horizon == 0;    // capacity-sized: surplus workgroups
        if (v.replay_horizon > 0) {
            // a horizon: each sequence sized for its rows now plus that many
            // appends (the merge launch marks a sequence the grid no longer
            // covers with NaN rows)
            std::vector<int32_t> r(v.rows);
            for (auto& x : r) {
                const int64_t n = static_cast<int64_t>(x) + v.replay_horizon;
                x = static_cast<int32_t>(n < a.row_limit ? n : a.row_limit);
            }
            a.n_chunks = chunks_for(r, a.chunk_rows);
        }
        // the device lengths may grow up to the row limit between replays
        a.one_chunk = per_seq <= 1 ? 1 : 0;
    } else {
        a.chunk_rows = chunk_rows ? chunk_rows
                                  : auto_chunk(v.rows, v.n_kv_heads, esz_of(v.dtype),
                                               kvdec::resident_attend_blocks(v.dtype, group), group,
                                               v.table != nullptr);
        a.n_chunks = chunks_for(v.rows, a.chunk_rows);
        a.need_merge = a.n_chunks > v.batch;   // some sequence has more than one chunk
        // the launch reads the lengths the grid was sized from
        a.one_chunk = a.n_chunks == v.batch ? 1 : 0;
        // equal lengths: the launch needs to read none of them to find its chunk
        bool equal = true;
        for (int32_t r : v.rows) equal = equal && r == v.rows[0];
        a.uniform = equal && !v.rows.empty() ? v.rows[0] : -1;
    }
}

// The merge launch planned on the host: an entry for every sequence that
// `rows` and chunk size T split over several chunks, whose partials start
// at base_slot + the prefix of the chunk counts.  False (and the device-side
// merge is used) when there are more than the plan holds.
bool plan_merge(const std::vector<int32_t>& rows, int32_t T, int64_t base_slot, bool cross,
                kvdec::MergePlanHost& mp)
{
    int64_t slot = base_slot;
    for (size_t b = 0; b < rows.size(); ++b) {
        const int64_t n = (static_cast<int64_t>(rows[b]) + T - 1) / T;
        const int64_t nch = n > 0 ? n : 1;
        if (nch > 1) {
            if (mp.n >= kvdec::kMaxMergeEntries || nch >= (1 << 24) || slot > INT32_MAX) return false;
            mp.plan.first[mp.n] = static_cast<int32_t>(slot);
            mp.plan.b[mp.n] = static_cast<int32_t>(b);
            mp.plan.nch[mp.n] = static_cast<int32_t>(nch) | (cross ? (1 << 24) : 0);
            ++mp.n;
        }
        slot += nch;
    }
    return true;
}

// Everything else of the launch over view v (the append fused into it, the
// paged layout), after plan_chunks.
void fill_args(const AttendView& v, const float* q, float scale, float* out, void* ws,
               const kvdec::PartialLayout& part, kvdec::AttendArgs& a)
{
    a.q = q;
    a.k = v.k;
    a.v = v.v;
    a.qscale = scale * 1.4426950408889634f;
    a.out = out;
    a.ws = ws;
    a.part = part;
    a.table = v.table;
    a.table_stride = v.table_stride;
    a.pshift = v.pshift;
    a.num_pages = v.num_pages;
    a.fresh_pages = v.fresh_pages;
    a.fused_lens = v.fused_lens;
    a.fused_device = v.fused_device;
    if (v.fused_device) a.need_merge = true;   // the merge launch bumps the lengths
    a.k_new = v.k_new;
    a.v_new = v.v_new;
    a.lens_out = v.lens_out;
    a.window = v.window;
}

// The placement of a host-fused launch's chunks on the CUs (see
// kvdec::Placement): only for the MFMA kernel (bf16, grouped heads), where
// the launch is one residency round with ragged chunks, the CU count is a
// multiple of the KV heads, and every position class gets at least two
// chunks.  A
// chunk's weight is its rows plus a fixed per-workgroup cost; the heaviest
// go first, each into the least-loaded class that has a position left
// (ties to the lower class and the earlier chunk, so the plan is a function
// of the lengths alone).
constexpr int64_t kPlaceFixedRows = 32;

bool plan_placement(const AttendView& v, int32_t group, const kvdec::AttendArgs& a,
                    kvdec::Placement& pl)
{
    // the MFMA kernel (bf16, grouped heads) takes a placement
    if (v.dtype != KVDEC_BF16 || group < 2 || a.uniform >= 0 || a.x_blocks > 0) return false;
    const int32_t Hkv = v.n_kv_heads;
    const int64_t P = a.n_chunks;
    if (!placeable(P, Hkv, kvdec::resident_attend_blocks(v.dtype, group))) return false;
    const int64_t classes = kvdec::device_cus() / Hkv;
    const int64_t per = (P + classes - 1) / classes;
    const int64_t npos = per * classes;
    // chunk weights and entries in chunk order (sequence by sequence, as the
    // kernels number them; a chunk's partial slot is its index in this order)
    const int64_t T = a.chunk_rows;
    if (v.batch > 512) return false;
    std::vector<std::pair<int64_t, int32_t>> w;
    std::vector<uint32_t> entry;
    w.reserve(static_cast<size_t>(P));
    entry.reserve(static_cast<size_t>(P));
    for (int32_t b = 0; b < v.batch; ++b) {
        const int64_t n = std::min<int64_t>(std::max<int32_t>(v.rows[b], 0), v.row_limit);
        const int64_t nch = n > 0 ? (n + T - 1) / T : 1;
        if (nch > 128 || static_cast<int64_t>(w.size()) + nch > P) return false;
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t rows = std::min(n, (c + 1) * T) - c * T;
            w.emplace_back(-(rows + kPlaceFixedRows), static_cast<int32_t>(w.size()));
            entry.push_back(kvdec::place_entry(static_cast<uint32_t>(b), static_cast<uint32_t>(c),
                                               static_cast<uint32_t>(nch),
                                               static_cast<uint32_t>(entry.size())));
        }
    }
    if (static_cast<int64_t>(w.size()) != P) return false;
    std::sort(w.begin(), w.end());
    using Load = std::pair<int64_t, int32_t>;      // (load, class)
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int32_t k = 0; k < classes; ++k) heap.emplace(0, k);
    std::vector<int32_t> filled(static_cast<size_t>(classes), 0);
    for (int64_t p = 0; p < npos; ++p) pl.pos[p] = kvdec::kNoChunk;
    for (const auto& item : w) {
        const Load top = heap.top();
        heap.pop();
        const int32_t k = top.second;
        pl.pos[k + classes * filled[k]] = entry[static_cast<size_t>(item.second)];
        if (++filled[k] < per) heap.emplace(top.first - item.first, k);
    }
    pl.n = static_cast<int32_t>(npos);
    return true;
}

int32_t attend_view(const AttendView& v, const float* q, int32_t n_q_heads, float scale,
                    int32_t chunk_rows, float* out, void* ws, size_t ws_bytes, void* stream)
{
    const int32_t rc = check_attend(v, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes);
    if (rc) return rc;
    const int32_t group = n_q_heads / v.n_kv_heads;
    kvdec::PartialLayout part = kvdec::partial_layout(v.max_chunks, n_q_heads, v.batch);
    kvdec::AttendArgs a;
    plan_chunks(v, group, chunk_rows, a);
    if (v.use_scratch) {
        // the partial slots this launch writes (one per workgroup along x and
        // query head) and the length snapshot, in the library's scratch
        part = kvdec::partial_layout(a.n_chunks, n_q_heads, v.batch);
        size_t avail = 0;
        const hipError_t e = kvdec::scratch_device_ptr(&ws, &avail);
        if (e != hipSuccess) return hip_fail(e, "device scratch address");
        if (part.bytes > avail)
            return fail(KVDEC_E_WORKSPACE, "this call needs %zu bytes of device scratch (%lld chunks x "
                        "%d query heads); the library holds %zu", part.bytes,
                        static_cast<long long>(a.n_chunks), n_q_heads, avail);
    }
    fill_args(v, q, scale, out, ws, part, a);
    // outside replay mode the host holds every length the launch reads
    kvdec::MergePlanHost mp;
    if (v.replay_chunk == 0 && !v.fused_device && a.need_merge &&
        plan_merge(v.rows, a.chunk_rows, 0, false, mp))
        a.merge_plan = &mp;
    kvdec::Placement pl;
    if (v.fused_lens && v.replay_chunk == 0 && plan_placement(v, group, a, pl)) a.placement = &pl;
    const hipError_t e = kvdec::launch_attend(v.dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    return KVDEC_OK;
}

AttendView view_of(const kvdec_cache* c)
{
    AttendView v;
    v.batch = c->d.batch;
    v.n_kv_heads = c->d.n_kv_heads;
    v.dtype = c->d.dtype;
    v.cap_pad = c->cap_pad;
    v.row_limit = c->d.window > 0 ? c->d.window : c->d.capacity;
    v.replay_chunk = c->replay_chunk;
    v.replay_horizon = c->replay_horizon;
    v.k = c->d.k;
    v.v = c->d.v;
    v.lens_dev = c->d.lens;
    v.rows = attended_rows(c);
    v.max_chunks = max_chunks(c);
    return v;
}

// Calls outside replay mode size their launches (and check capacity) from
// the host mirror, so they need it to match the device lengths.
int32_t check_mirror(const kvdec_cache* c)
{
    if (c->replay_chunk == 0 && !c->lens_known)
        return fail(KVDEC_E_INVALID, "lengths unknown after leaving replay mode: set them with "
                    "kvdec_reset_lens (or kvdec_seed, kvdec_append_attend_at) first");
    return KVDEC_OK;
}

int32_t attend_common(const kvdec_cache* c, const float* q, int32_t n_q_heads, float scale,
                      int32_t chunk_rows, float* out, void* ws, size_t ws_bytes, void* stream)
{
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    const int32_t rc = check_mirror(c);
    if (rc) return rc;
    return attend_view(view_of(c), q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
}

int32_t check_append(const kvdec_cache* c, const void* k_new, const void* v_new)
{
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    if (c->d.is_static) return fail(KVDEC_E_STATIC, "append on a static (encoder) cache");
    const int32_t rc = check_mirror(c);
    if (rc) return rc;
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(KVDEC_E_INVALID, "k_new and v_new must be non-NULL, 16-byte aligned device pointers");
    for (int32_t b = 0; b < c->d.batch && c->replay_chunk == 0; ++b) {
        if (c->d.window == 0 && c->lens[b] + 1 > c->d.capacity)
            return fail(KVDEC_E_OVERFLOW, "cache overflow: sequence %d holds %d + 1 > %d", b,
                        c->lens[b], c->d.capacity);
        if (c->lens[b] == INT32_MAX)
            return fail(KVDEC_E_OVERFLOW, "token count of sequence %d would overflow int32", b);
    }
    return KVDEC_OK;
}

// Checks of an append at explicit positions lens_host (kvdec_append_attend_at
// and the layer step given positions); the positions go to `pre`.
int32_t check_positions(const kvdec_cache* c, const int32_t* lens_host, const void* k_new,
                        const void* v_new, std::vector<int32_t>& pre)
{
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    const int32_t rc = check_lens(lens_host, c->d.batch, c->d.capacity, c->d.window);
    if (rc) return rc;
    pre.assign(lens_host, lens_host + c->d.batch);
    for (int32_t b = 0; b < c->d.batch; ++b) {
        if (c->d.window == 0 && pre[b] >= c->d.capacity)
            return fail(KVDEC_E_OVERFLOW, "cache overflow: sequence %d at position %d, capacity %d",
                        b, pre[b], c->d.capacity);
        if (pre[b] == INT32_MAX)
            return fail(KVDEC_E_OVERFLOW, "token count of sequence %d would overflow int32", b);
    }
    if (c->d.is_static) return fail(KVDEC_E_STATIC, "append on a static (encoder) cache");
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(KVDEC_E_INVALID, "k_new and v_new must be non-NULL, 16-byte aligned device pointers");
    return KVDEC_OK;
}

}  // namespace

namespace {

// The fused decode step from pre-append lengths `pre` (the host mirror, or
// the positions kvdec_append_attend_at was given).  Arguments are checked by
// the callers; `set_device` first writes `pre` to the device lengths where
// the launch reads them from there.
int32_t append_attend_from(kvdec_cache* c, const std::vector<int32_t>& pre, bool set_device,
                           const void* k_new, const void* v_new, const float* q,
                           int32_t n_q_heads, float scale, int32_t chunk_rows, float* out,
                           void* ws, size_t ws_bytes, void* stream, bool use_scratch = false)
{
    AttendView v = view_of(c);
    v.use_scratch = use_scratch;
    // rows attended after the append
    for (size_t b = 0; b < pre.size(); ++b) {
        const int64_t n = static_cast<int64_t>(pre[b]) + 1;
        v.rows[b] = static_cast<int32_t>(c->d.window > 0 && n > c->d.window ? c->d.window : n);
    }
    int32_t rc = check_attend(v, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes);
    if (rc) return rc;
    if (c->d.batch > KVDEC_MAX_FUSED_BATCH || c->replay_chunk > 0) {
        // attend + merge launch; the lengths are read from (and bumped on) the device
        if (set_device) {
            const hipError_t e = kvdec::launch_set_lens(c->d.lens, pre.data(), c->d.batch,
                                                        static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "set lengths");
            c->lens = pre;             // mirror and device agree even if the attend launch fails
            c->lens_known = true;
        }
        v.fused_device = true;
    } else {
        v.fused_lens = pre.data();     // one launch; pre-append lengths by value
    }
    v.k_new = k_new;
    v.v_new = v_new;
    v.lens_out = c->d.lens;
    v.window = c->d.window;
    rc = attend_view(v, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
    if (rc) return rc;
    c->lens = pre;
    for (auto& l : c->lens) ++l;
    if (set_device) c->lens_known = true;     // the positions came from the caller
    return KVDEC_OK;
}

}  // namespace

namespace {

AttendView paged_view_of(const kvdec_paged* p)
{
    const int64_t cap = static_cast<int64_t>(p->d.max_pages_per_seq) * p->d.page_rows;
    AttendView v;
    v.batch = p->d.batch;
    v.n_kv_heads = p->d.n_kv_heads;
    v.dtype = p->d.dtype;
    v.cap_pad = 0;
    v.row_limit = static_cast<int32_t>(cap);
    v.replay_chunk = p->replay_chunk;
    v.replay_horizon = p->replay_horizon;
    v.k = p->d.k_pages;
    v.v = p->d.v_pages;
    v.lens_dev = p->d.lens;
    v.rows = p->lens;
    v.max_chunks = p->d.batch * ((cap + KVDEC_MIN_CHUNK - 1) / KVDEC_MIN_CHUNK);
    v.table = p->d.block_table;
    v.table_stride = p->d.max_pages_per_seq;
    v.pshift = p->pshift;
    v.num_pages = p->d.num_pages;
    return v;
}

// Pages for the sequences whose next row starts a page (sequence order,
// lowest-numbered first), installed in the host mirror of the table;
// fresh[b] = the page, or -1.  The caller has checked that enough are free.
std::vector<int32_t> take_fresh_pages(kvdec_paged* p)
{
    const int32_t P = p->d.page_rows;
    std::vector<int32_t> fresh(p->d.batch, -1);
    for (int32_t b = 0; b < p->d.batch; ++b)
        if (p->lens[b] % P == 0) {
            fresh[b] = p->free_pages.back();
            p->free_pages.pop_back();
            p->table[static_cast<size_t>(b) * p->d.max_pages_per_seq + p->lens[b] / P] = fresh[b];
        }
    return fresh;
}

void return_fresh_pages(kvdec_paged* p, const std::vector<int32_t>& fresh)
{
    const int32_t P = p->d.page_rows;
    for (int32_t b = p->d.batch - 1; b >= 0; --b)
        if (fresh[b] >= 0) {
            p->table[static_cast<size_t>(b) * p->d.max_pages_per_seq + p->lens[b] / P] = -1;
            p->free_pages.push_back(fresh[b]);
        }
}

// Calls outside replay mode size launches and take pages from the host
// mirror, so they need it to match the device lengths.
int32_t check_paged_mirror(const kvdec_paged* p)
{
    if (p->replay_chunk == 0 && !p->lens_known)
        return fail(KVDEC_E_INVALID, "lengths unknown after leaving replay mode: set them with "
                    "kvdec_paged_truncate first");
    return KVDEC_OK;
}

// Return the pages of sequence b past its first `keep` to the pool (host
// mirror), and collect their table entries.  In replay mode they are set to
// -1 on the device at once, so that an append that reads its page from the
// table never finds one another sequence now holds; outside replay mode
// nothing reads an entry past a sequence's pages, and entering replay mode
// clears them all.
void free_pages_past(kvdec_paged* p, int32_t b, int32_t keep, std::vector<int32_t>& cleared)
{
    const size_t base = static_cast<size_t>(b) * p->d.max_pages_per_seq;
    const int32_t held = (p->lens[b] + p->d.page_rows - 1) / p->d.page_rows;
    for (int32_t i = held - 1; i >= keep; --i) {
        p->free_pages.push_back(p->table[base + i]);
        p->table[base + i] = -1;
        cleared.push_back(static_cast<int32_t>(base) + i);
    }
}

hipError_t clear_entries(kvdec_paged* p, const std::vector<int32_t>& cleared, void* stream)
{
    if (p->replay_chunk == 0) return hipSuccess;
    const std::vector<int32_t> minus(cleared.size(), -1);
    return kvdec::launch_table_write(p->d.block_table, cleared.data(), minus.data(),
                                     static_cast<int32_t>(cleared.size()),
                                     static_cast<hipStream_t>(stream));
}

// Capacity and pool checks of a paged append (nothing changes on failure).
// In replay mode the pages were given ahead (kvdec_paged_prepare) and the
// device drops a row that has none, so there is nothing to check here.
int32_t check_paged_append(const kvdec_paged* p, const void* k_new, const void* v_new)
{
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(KVDEC_E_INVALID, "k_new and v_new must be non-NULL, 16-byte aligned device pointers");
    const int32_t rc = check_paged_mirror(p);
    if (rc || p->replay_chunk > 0) return rc;
    const int32_t P = p->d.page_rows;
    const int64_t cap = static_cast<int64_t>(p->d.max_pages_per_seq) * P;
    int32_t needed = 0;
    for (int32_t b = 0; b < p->d.batch; ++b) {
        if (p->lens[b] + 1 > cap)
            return fail(KVDEC_E_OVERFLOW, "cache overflow: sequence %d holds %d + 1 > %lld", b,
                        p->lens[b], static_cast<long long>(cap));
        if (p->lens[b] % P == 0) ++needed;
    }
    if (needed > static_cast<int32_t>(p->free_pages.size()))
        return fail(KVDEC_E_OVERFLOW, "page pool exhausted: %d new pages needed, %zu free", needed,
                    p->free_pages.size());
    return KVDEC_OK;
}

}  // namespace

extern "C" {

int32_t kvdec_padded_capacity(int32_t capacity)
{
    if (capacity < 1) return 0;
    const int64_t p = (static_cast<int64_t>(capacity) + KVDEC_ROW_ALIGN - 1) / KVDEC_ROW_ALIGN *
                      KVDEC_ROW_ALIGN;
    return p > INT32_MAX ? 0 : static_cast<int32_t>(p);
}

int32_t kvdec_cache_create(const kvdec_cache_desc* desc, const int32_t* lens_host, void* stream,
                           kvdec_cache** out)
{
    g_err.clear();
    if (!desc || !out) return fail(KVDEC_E_INVALID, "desc and out must not be NULL");
    *out = nullptr;
    const kvdec_cache_desc& d = *desc;
    if (d.batch < 1 || d.n_kv_heads < 1 || d.capacity < 1)
        return fail(KVDEC_E_INVALID, "batch, n_kv_heads and capacity must be >= 1");
    if (d.head_dim != KVDEC_HEAD_DIM)
        return fail(KVDEC_E_SHAPE, "head_dim must be %d, got %d", KVDEC_HEAD_DIM, d.head_dim);
    if (d.dtype != KVDEC_F32 && d.dtype != KVDEC_BF16)
        return fail(KVDEC_E_INVALID, "unknown dtype %d", d.dtype);
    if (d.is_static != 0 && d.is_static != 1) return fail(KVDEC_E_INVALID, "is_static must be 0 or 1");
    if (d.window != 0 && d.window != d.capacity)
        return fail(KVDEC_E_SHAPE, "window must be 0 or equal to capacity (%d), got %d", d.capacity,
                    d.window);
    if (d.window != 0 && d.is_static)
        return fail(KVDEC_E_INVALID, "a static (encoder) cache cannot be a sliding-window ring");
    if (d.reserved0 != 0) return fail(KVDEC_E_INVALID, "reserved0 must be 0");
    if (!aligned16(d.k) || !aligned16(d.v) || !aligned16(d.lens))
        return fail(KVDEC_E_INVALID, "k, v and lens must be non-NULL, 16-byte aligned device pointers");
    const int32_t cap_pad = kvdec_padded_capacity(d.capacity);
    if (cap_pad == 0) return fail(KVDEC_E_SHAPE, "capacity %d too large", d.capacity);
    int32_t rc = check_lens(lens_host, d.batch, d.capacity, d.window);
    if (rc) return rc;
    kvdec_cache* c = new kvdec_cache;
    c->d = d;
    c->cap_pad = cap_pad;
    c->lens.assign(lens_host, lens_host + d.batch);
    const hipError_t e = kvdec::launch_set_lens(d.lens, lens_host, d.batch,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "set lengths");
    }
    *out = c;
    return KVDEC_OK;
}

void kvdec_cache_destroy(kvdec_cache* cache) { delete cache; }

int32_t kvdec_reset_lens(kvdec_cache* c, const int32_t* lens_host, void* stream)
{
    g_err.clear();
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    int32_t rc = check_lens(lens_host, c->d.batch, c->d.capacity, c->d.window);
    if (rc) return rc;
    const hipError_t e = kvdec::launch_set_lens(c->d.lens, lens_host, c->d.batch,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set lengths");
    c->lens.assign(lens_host, lens_host + c->d.batch);
    c->lens_known = true;
    return KVDEC_OK;
}

int32_t kvdec_get_lens(const kvdec_cache* c, int32_t* lens_out)
{
    g_err.clear();
    if (!c || !lens_out) return fail(KVDEC_E_INVALID, "cache and lens_out must not be NULL");
    if (!c->lens_known)
        return fail(KVDEC_E_INVALID, "lengths unknown after leaving replay mode (kvdec_reset_lens sets them)");
    std::memcpy(lens_out, c->lens.data(), sizeof(int32_t) * c->lens.size());
    return KVDEC_OK;
}

int32_t kvdec_seed(kvdec_cache* c, const void* k_tok, const void* v_tok, int32_t rows, void* stream)
{
    g_err.clear();
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    if (rows < 0 || rows > c->d.capacity)
        return fail(KVDEC_E_SHAPE, "rows %d outside [0, capacity %d]", rows, c->d.capacity);
    if (rows > 0 && (!aligned16(k_tok) || !aligned16(v_tok)))
        return fail(KVDEC_E_INVALID, "k_tok and v_tok must be non-NULL, 16-byte aligned device pointers");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kvdec::launch_seed(c->d.dtype, c->d.k, c->d.v, k_tok, v_tok, c->d.batch, rows,
                                      c->d.n_kv_heads, c->cap_pad, s);
    if (e != hipSuccess) return hip_fail(e, "seed launch");
    std::vector<int32_t> l(c->d.batch, rows);
    e = kvdec::launch_set_lens(c->d.lens, l.data(), c->d.batch, s);
    if (e != hipSuccess) return hip_fail(e, "set lengths");
    c->lens = l;
    c->lens_known = true;
    return KVDEC_OK;
}

int32_t kvdec_append(kvdec_cache* c, const void* k_new, const void* v_new, void* stream)
{
    g_err.clear();
    const int32_t rc = check_append(c, k_new, v_new);
    if (rc) return rc;
    const hipError_t e = kvdec::launch_append(c->d.dtype, c->d.k, c->d.v, k_new, v_new, c->d.lens,
                                              c->d.batch, c->d.n_kv_heads, c->d.capacity,
                                              c->cap_pad, c->d.window,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
    for (auto& l : c->lens) ++l;
    return KVDEC_OK;
}

int32_t kvdec_append_slide(kvdec_cache* c, const void* k_new, const void* v_new, int32_t overlap,
                           int32_t* slid_out, void* stream)
{
    g_err.clear();
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    if (c->d.is_static) return fail(KVDEC_E_STATIC, "append on a static (encoder) cache");
    if (c->d.window != 0)
        return fail(KVDEC_E_INVALID, "a sliding-window ring already keeps the last window rows; "
                    "kvdec_append_slide needs a linear cache");
    if (overlap < 0) return fail(KVDEC_E_INVALID, "overlap %d must be >= 0", overlap);
    const int32_t rc = check_mirror(c);
    if (rc) return rc;
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(KVDEC_E_INVALID, "k_new and v_new must be non-NULL, 16-byte aligned device pointers");
    const int32_t keep = overlap < c->d.capacity / 2 ? overlap : c->d.capacity / 2;
    const hipError_t e = kvdec::launch_append_slide(c->d.dtype, c->d.k, c->d.v, k_new, v_new, c->d.lens,
                                                    c->d.batch, c->d.n_kv_heads, c->d.capacity,
                                                    c->cap_pad, keep, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
    for (int32_t b = 0; b < c->d.batch; ++b) {
        const bool slide = c->lens[b] + 1 > c->d.capacity;
        if (slide) c->lens[b] = keep;
        if (slid_out) slid_out[b] = slide ? 1 : 0;
        ++c->lens[b];
    }
    return KVDEC_OK;
}

int32_t kvdec_append_rope(kvdec_cache* c, const void* k_new, const void* v_new, float theta,
                          const float* q, float* q_rot, int32_t n_q_heads, void* stream)
{
    g_err.clear();
    const int32_t rc = check_append(c, k_new, v_new);
    if (rc) return rc;
    if (!(theta > 0.f) || !std::isfinite(theta))
        return fail(KVDEC_E_INVALID, "theta must be a positive finite number");
    if ((q == nullptr) != (q_rot == nullptr))
        return fail(KVDEC_E_INVALID, "q and q_rot must both be given or both be NULL");
    if (q) {
        if (!aligned16(q) || !aligned16(q_rot))
            return fail(KVDEC_E_INVALID, "q and q_rot must be 16-byte aligned device pointers");
        if (n_q_heads <= 0 || n_q_heads % c->d.n_kv_heads != 0)
            return fail(KVDEC_E_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                        n_q_heads, c->d.n_kv_heads);
    }
    const hipError_t e = kvdec::launch_append_rope(
        c->d.dtype, c->d.k, c->d.v, k_new, v_new, c->d.lens, c->d.batch, c->d.n_kv_heads,
        c->d.capacity, c->cap_pad, c->d.window, q, q_rot, q ? n_q_heads : 0,
        static_cast<double>(theta), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
    for (auto& l : c->lens) ++l;
    return KVDEC_OK;
}

size_t kvdec_workspace_bytes(const kvdec_cache* c, int32_t n_q_heads)
{
    if (!c || n_q_heads <= 0) return 0;
    return kvdec::partial_layout(max_chunks(c), n_q_heads, c->d.batch).bytes;
}

int32_t kvdec_attend_self(const kvdec_cache* c, const float* q, int32_t n_q_heads, float scale,
                          int32_t chunk_rows, float* out, void* ws, size_t ws_bytes, void* stream)
{
    g_err.clear();
    if (c && c->d.is_static)
        return fail(KVDEC_E_STATIC, "self-attention on a static (encoder) cache; use kvdec_attend_cross");
    return attend_common(c, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
}

int32_t kvdec_attend_cross(const kvdec_cache* c, const float* q, int32_t n_q_heads, float scale,
                           int32_t chunk_rows, float* out, void* ws, size_t ws_bytes, void* stream)
{
    g_err.clear();
    if (c && !c->d.is_static)
        return fail(KVDEC_E_STATIC, "cross-attention needs a static (encoder) cache");
    return attend_common(c, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
}

int32_t kvdec_set_replay_mode(kvdec_cache* c, int32_t chunk_rows)
{
    g_err.clear();
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    if (chunk_rows == KVDEC_REPLAY_AUTO) {
        // the automatic choice for the current lengths, with the query-head
        // group of a plain MHA call (the grid shape does not depend on it)
        c->replay_chunk = auto_chunk(attended_rows(c), c->d.n_kv_heads, esz_of(c->d.dtype),
                                     kvdec::resident_attend_blocks(c->d.dtype, 1));
        return KVDEC_OK;
    }
    if (chunk_rows != 0 && (chunk_rows < KVDEC_MIN_CHUNK || chunk_rows > KVDEC_MAX_CHUNK ||
                            chunk_rows % 64 != 0))
        return fail(KVDEC_E_INVALID, "chunk_rows %d must be 0, KVDEC_REPLAY_AUTO or a multiple of "
                    "64 in [%d, %d]", chunk_rows, KVDEC_MIN_CHUNK, KVDEC_MAX_CHUNK);
    // leaving replay mode: replays may have appended on the device, which
    // the mirror does not see (a static cache takes no appends)
    if (chunk_rows == 0 && c->replay_chunk > 0 && !c->d.is_static) c->lens_known = false;
    c->replay_chunk = chunk_rows;
    return KVDEC_OK;
}

int32_t kvdec_set_replay_horizon(kvdec_cache* c, int32_t tokens)
{
    g_err.clear();
    if (!c) return fail(KVDEC_E_INVALID, "cache handle is NULL");
    if (tokens < 0) return fail(KVDEC_E_INVALID, "tokens %d must be >= 0", tokens);
    c->replay_horizon = tokens;
    return KVDEC_OK;
}


int32_t kvdec_paged_create(const kvdec_paged_desc* desc, void* stream, kvdec_paged** out)
{
    g_err.clear();
    if (!desc || !out) return fail(KVDEC_E_INVALID, "desc and out must not be NULL");
    *out = nullptr;
    const kvdec_paged_desc& d = *desc;
    if (d.batch < 1 || d.n_kv_heads < 1 || d.num_pages < 1 || d.max_pages_per_seq < 1)
        return fail(KVDEC_E_INVALID, "batch, n_kv_heads, num_pages and max_pages_per_seq must be >= 1");
    if (d.head_dim != KVDEC_HEAD_DIM)
        return fail(KVDEC_E_SHAPE, "head_dim must be %d, got %d", KVDEC_HEAD_DIM, d.head_dim);
    if (d.dtype != KVDEC_F32 && d.dtype != KVDEC_BF16)
        return fail(KVDEC_E_INVALID, "unknown dtype %d", d.dtype);
    int32_t pshift = 0;
    while ((1 << pshift) < d.page_rows && pshift < 13) ++pshift;
    if (d.page_rows < 16 || d.page_rows > KVDEC_MAX_CHUNK || (1 << pshift) != d.page_rows)
        return fail(KVDEC_E_SHAPE, "page_rows must be a power of two in [16, %d], got %d",
                    KVDEC_MAX_CHUNK, d.page_rows);
    if (static_cast<int64_t>(d.max_pages_per_seq) * d.page_rows > INT32_MAX / 2 ||
        static_cast<int64_t>(d.max_pages_per_seq) * d.batch > INT32_MAX)
        return fail(KVDEC_E_SHAPE, "max_pages_per_seq * page_rows or * batch too large");
    if (d.reserved0 != 0) return fail(KVDEC_E_INVALID, "reserved0 must be 0");
    if (!aligned16(d.k_pages) || !aligned16(d.v_pages) || !aligned16(d.block_table) ||
        !aligned16(d.lens))
        return fail(KVDEC_E_INVALID,
                    "k_pages, v_pages, block_table and lens must be non-NULL, 16-byte aligned device pointers");
    kvdec_paged* p = new kvdec_paged;
    p->d = d;
    p->pshift = pshift;
    p->lens.assign(d.batch, 0);
    p->table.assign(static_cast<size_t>(d.batch) * d.max_pages_per_seq, -1);
    p->free_pages.reserve(d.num_pages);
    for (int32_t i = d.num_pages - 1; i >= 0; --i) p->free_pages.push_back(i);   // pops 0, 1, 2, ...
    hipError_t e = kvdec::launch_set_lens(d.lens, p->lens.data(), d.batch,
                                          static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = kvdec::launch_fill_i32(d.block_table, static_cast<int64_t>(d.batch) * d.max_pages_per_seq,
                                   -1, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "set lengths and block table");
    }
    *out = p;
    return KVDEC_OK;
}

void kvdec_paged_destroy(kvdec_paged* p) { delete p; }

int32_t kvdec_paged_append(kvdec_paged* p, const void* k_new, const void* v_new, void* stream)
{
    g_err.clear();
    const int32_t rc = check_paged_append(p, k_new, v_new);
    if (rc) return rc;
    if (p->replay_chunk > 0) {
        // pages were given ahead; the mirror already counts the prepared rows
        const std::vector<int32_t> none(p->d.batch, -1);
        const hipError_t e = kvdec::launch_paged_append(
            p->d.dtype, p->d.k_pages, p->d.v_pages, k_new, v_new, p->d.lens, p->d.block_table,
            p->d.max_pages_per_seq, p->d.batch, p->d.n_kv_heads, p->pshift, p->d.num_pages,
            none.data(), true, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? KVDEC_OK : hip_fail(e, "paged append launch");
    }
    // take pages, install them in the host mirror, launch; on a launch
    // failure give everything back
    const std::vector<int32_t> fresh = take_fresh_pages(p);
    const hipError_t e = kvdec::launch_paged_append(
        p->d.dtype, p->d.k_pages, p->d.v_pages, k_new, v_new, p->d.lens, p->d.block_table,
        p->d.max_pages_per_seq, p->d.batch, p->d.n_kv_heads, p->pshift, p->d.num_pages, fresh.data(),
        false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        return_fresh_pages(p, fresh);
        return hip_fail(e, "paged append launch");
    }
    for (auto& l : p->lens) ++l;
    return KVDEC_OK;
}

int32_t kvdec_paged_release(kvdec_paged* p, int32_t seq, void* stream)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (seq < 0 || seq >= p->d.batch)
        return fail(KVDEC_E_INVALID, "sequence %d outside [0, %d)", seq, p->d.batch);
    const int32_t zero = 0;
    const hipError_t e = kvdec::launch_set_lens(p->d.lens + seq, &zero, 1,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set lengths");
    std::vector<int32_t> cleared;
    free_pages_past(p, seq, 0, cleared);
    p->lens[seq] = 0;
    const hipError_t e2 = clear_entries(p, cleared, stream);
    return e2 == hipSuccess ? KVDEC_OK : hip_fail(e2, "block table write");
}

int32_t kvdec_paged_reserve(kvdec_paged* p, int32_t seq, int32_t len, void* stream)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (seq < 0 || seq >= p->d.batch)
        return fail(KVDEC_E_INVALID, "sequence %d outside [0, %d)", seq, p->d.batch);
    const int32_t rc = check_paged_mirror(p);
    if (rc) return rc;
    if (p->lens[seq] != 0)
        return fail(KVDEC_E_INVALID, "sequence %d is not empty (%d rows)", seq, p->lens[seq]);
    const int64_t cap = static_cast<int64_t>(p->d.max_pages_per_seq) * p->d.page_rows;
    if (len < 0 || len > cap)
        return fail(KVDEC_E_OVERFLOW, "length %d outside [0, %lld]", len, static_cast<long long>(cap));
    const int32_t n = (len + p->d.page_rows - 1) / p->d.page_rows;
    if (n > static_cast<int32_t>(p->free_pages.size()))
        return fail(KVDEC_E_OVERFLOW, "page pool exhausted: %d pages needed, %zu free", n,
                    p->free_pages.size());
    std::vector<int32_t> pages(n);
    for (int32_t i = 0; i < n; ++i) {
        pages[i] = p->free_pages.back();
        p->free_pages.pop_back();
    }
    const hipError_t e = kvdec::launch_paged_reserve(p->d.block_table, p->d.max_pages_per_seq,
                                                     p->d.lens, seq, pages.data(), n, len,
                                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        for (int32_t i = n - 1; i >= 0; --i) p->free_pages.push_back(pages[i]);
        return hip_fail(e, "paged reserve launch");
    }
    const size_t base = static_cast<size_t>(seq) * p->d.max_pages_per_seq;
    for (int32_t i = 0; i < n; ++i) p->table[base + i] = pages[i];
    p->lens[seq] = len;
    return KVDEC_OK;
}

int32_t kvdec_paged_truncate(kvdec_paged* p, const int32_t* lens_host, void* stream)
{
    g_err.clear();
    if (!p || !lens_host) return fail(KVDEC_E_INVALID, "handle and lens_host must not be NULL");
    // a known length only shrinks; after replay mode a length may be
    // anything the sequence's pages hold (replays may have appended more or
    // fewer rows than were prepared)
    const int32_t P = p->d.page_rows;
    for (int32_t b = 0; b < p->d.batch; ++b) {
        const int64_t limit = p->lens_known ? p->lens[b]
                                            : static_cast<int64_t>((p->lens[b] + P - 1) / P) * P;
        if (lens_host[b] < 0 || lens_host[b] > limit)
            return fail(KVDEC_E_SHAPE, "new length %d of sequence %d outside [0, %lld]", lens_host[b],
                        b, static_cast<long long>(limit));
    }
    const hipError_t e = kvdec::launch_set_lens(p->d.lens, lens_host, p->d.batch,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set lengths");
    std::vector<int32_t> cleared;
    for (int32_t b = 0; b < p->d.batch; ++b) {
        free_pages_past(p, b, (lens_host[b] + P - 1) / P, cleared);
        p->lens[b] = lens_host[b];
    }
    p->lens_known = true;
    const hipError_t e2 = clear_entries(p, cleared, stream);
    return e2 == hipSuccess ? KVDEC_OK : hip_fail(e2, "block table write");
}

int32_t kvdec_paged_get_lens(const kvdec_paged* p, int32_t* lens_out)
{
    g_err.clear();
    if (!p || !lens_out) return fail(KVDEC_E_INVALID, "handle and lens_out must not be NULL");
    const int32_t rc = check_paged_mirror(p);
    if (rc) return rc;
    std::memcpy(lens_out, p->lens.data(), sizeof(int32_t) * p->lens.size());
    return KVDEC_OK;
}

int32_t kvdec_paged_get_table(const kvdec_paged* p, int32_t* table_out)
{
    g_err.clear();
    if (!p || !table_out) return fail(KVDEC_E_INVALID, "handle and table_out must not be NULL");
    std::memcpy(table_out, p->table.data(), sizeof(int32_t) * p->table.size());
    return KVDEC_OK;
}

int32_t kvdec_paged_free_pages(const kvdec_paged* p)
{
    return p ? static_cast<int32_t>(p->free_pages.size()) : -1;
}

size_t kvdec_paged_workspace_bytes(const kvdec_paged* p, int32_t n_q_heads)
{
    if (!p || n_q_heads <= 0) return 0;
    const int64_t cap = static_cast<int64_t>(p->d.max_pages_per_seq) * p->d.page_rows;
    return kvdec::partial_layout(p->d.batch * ((cap + KVDEC_MIN_CHUNK - 1) / KVDEC_MIN_CHUNK),
                                 n_q_heads, p->d.batch).bytes;
}

int32_t kvdec_paged_attend(const kvdec_paged* p, const float* q, int32_t n_q_heads, float scale,
                           int32_t chunk_rows, float* out, void* ws, size_t ws_bytes, void* stream)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    const int32_t rc = check_paged_mirror(p);
    if (rc) return rc;
    return attend_view(paged_view_of(p), q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
}

int32_t kvdec_paged_append_attend(kvdec_paged* p, const void* k_new, const void* v_new,
                                  const float* q, int32_t n_q_heads, float scale, int32_t chunk_rows,
                                  float* out, void* ws, size_t ws_bytes, void* stream)
{
    g_err.clear();
    int32_t rc = check_paged_append(p, k_new, v_new);
    if (rc) return rc;
    AttendView v = paged_view_of(p);
    for (auto& r : v.rows) ++r;                  // rows attended after the append
    rc = check_attend(v, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes);
    if (rc) return rc;
    if (p->replay_chunk > 0) {
        // replay mode: the attend launch reads the pre-append lengths from the
        // device and stores each new row in the page the table already holds
        // for it; the merge launch bumps the lengths
        AttendView r = paged_view_of(p);
        r.fused_device = true;
        r.k_new = k_new;
        r.v_new = v_new;
        r.lens_out = p->d.lens;
        return attend_view(r, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
    }
    if (p->d.batch > KVDEC_MAX_PAGED_FUSED_BATCH) {
        // two launches: the paged append, then the attend over the new lengths
        rc = kvdec_paged_append(p, k_new, v_new, stream);
        if (rc) return rc;
        return attend_view(paged_view_of(p), q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes,
                           stream);
    }
    const std::vector<int32_t> pre = p->lens;
    const std::vector<int32_t> fresh = take_fresh_pages(p);
    v.fused_lens = pre.data();
    v.fresh_pages = fresh.data();
    v.k_new = k_new;
    v.v_new = v_new;
    v.lens_out = p->d.lens;
    rc = attend_view(v, q, n_q_heads, scale, chunk_rows, out, ws, ws_bytes, stream);
    if (rc) {
        return_fresh_pages(p, fresh);
        return rc;
    }
    for (auto& l : p->lens) ++l;
    return KVDEC_OK;
}

int32_t kvdec_paged_set_replay_mode(kvdec_paged* p, int32_t chunk_rows, void* stream)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (chunk_rows != 0 && chunk_rows != KVDEC_REPLAY_AUTO &&
        (chunk_rows < KVDEC_MIN_CHUNK || chunk_rows > KVDEC_MAX_CHUNK || chunk_rows % 64 != 0))
        return fail(KVDEC_E_INVALID, "chunk_rows %d must be 0, KVDEC_REPLAY_AUTO or a multiple of "
                    "64 in [%d, %d]", chunk_rows, KVDEC_MIN_CHUNK, KVDEC_MAX_CHUNK);
    if (chunk_rows != 0 && p->replay_chunk == 0) {
        const int32_t rc = check_paged_mirror(p);   // prepare counts from exact lengths
        if (rc) return rc;
        // every entry past a sequence's pages becomes -1 on the device
        std::vector<int32_t> held(p->d.batch);
        for (int32_t b = 0; b < p->d.batch; ++b)
            held[b] = (p->lens[b] + p->d.page_rows - 1) / p->d.page_rows;
        const hipError_t e = kvdec::launch_table_clear_tail(p->d.block_table, p->d.max_pages_per_seq,
                                                            held.data(), p->d.batch,
                                                            static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "block table write");
    }
    if (chunk_rows == KVDEC_REPLAY_AUTO) {
        p->replay_chunk = auto_chunk(p->lens, p->d.n_kv_heads, esz_of(p->d.dtype),
                                     kvdec::resident_attend_blocks(p->d.dtype, 1));
        return KVDEC_OK;
    }
    // leaving replay mode: the mirror counts prepared rows, which replays may
    // not all have appended
    if (chunk_rows == 0 && p->replay_chunk > 0) p->lens_known = false;
    p->replay_chunk = chunk_rows;
    return KVDEC_OK;
}

int32_t kvdec_paged_set_replay_horizon(kvdec_paged* p, int32_t tokens)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (tokens < 0) return fail(KVDEC_E_INVALID, "tokens %d must be >= 0", tokens);
    p->replay_horizon = tokens;
    return KVDEC_OK;
}

int32_t kvdec_paged_prepare(kvdec_paged* p, int32_t n_tokens, void* stream)
{
    g_err.clear();
    if (!p) return fail(KVDEC_E_INVALID, "paged cache handle is NULL");
    if (p->replay_chunk == 0)
        return fail(KVDEC_E_INVALID, "kvdec_paged_prepare needs replay mode (outside it appends "
                    "take their own pages)");
    if (n_tokens < 0) return fail(KVDEC_E_INVALID, "n_tokens %d must be >= 0", n_tokens);
    const int32_t P = p->d.page_rows;
    const int64_t cap = static_cast<int64_t>(p->d.max_pages_per_seq) * P;
    int64_t needed = 0;
    for (int32_t b = 0; b < p->d.batch; ++b) {
        const int64_t want = static_cast<int64_t>(p->lens[b]) + n_tokens;
        if (want > cap)
            return fail(KVDEC_E_OVERFLOW, "cache overflow: sequence %d holds %d + %d > %lld", b,
                        p->lens[b], n_tokens, static_cast<long long>(cap));
        needed += (want + P - 1) / P - (p->lens[b] + P - 1) / P;
    }
    if (needed > static_cast<int64_t>(p->free_pages.size()))
        return fail(KVDEC_E_OVERFLOW, "page pool exhausted: %lld new pages needed, %zu free",
                    static_cast<long long>(needed), p->free_pages.size());
    // pages in sequence order, lowest-numbered first, as appends take them
    std::vector<int32_t> idx, val;
    for (int32_t b = 0; b < p->d.batch; ++b) {
        const size_t base = static_cast<size_t>(b) * p->d.max_pages_per_seq;
        const int32_t from = (p->lens[b] + P - 1) / P;
        const int32_t to = static_cast<int32_t>((static_cast<int64_t>(p->lens[b]) + n_tokens + P - 1) / P);
        for (int32_t i = from; i < to; ++i) {
            const int32_t page = p->free_pages.back();
            p->free_pages.pop_back();
            p->table[base + i] = page;
            idx.push_back(static_cast<int32_t>(base) + i);
            val.push_back(page);
        }
    }
    const hipError_t e = kvdec::launch_table_write(p->d.block_table, idx.data(), val.data(),
                                                   static_cast<int32_t>(idx.size()),
                                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        for (size_t k = idx.size(); k-- > 0;) {
            p->table[idx[k]] = -1;
            p->free_pages.push_back(val[k]);
        }
        return hip_fail(e, "block table write");
    }
    for (auto& l : p->lens) l += n_tokens;
    return KVDEC_OK;
}

int32_t kvdec_append_attend(kvdec_cache* c, const void* k_new, const void* v_new, const float* q,
                            int32_t n_q_heads, float scale, int32_t chunk_rows, float* out, void* ws,
                            size_t ws_bytes, void* stream)
{
    g_err.clear();
    const int32_t rc = check_append(c, k_new, v_new);
    if (rc) return rc;
    const std::vector<int32_t> pre = c->lens;
    return append_attend_from(c, pre, false, k_new, v_new, q, n_q_heads, scale, chunk_rows, out,
                              ws, ws_bytes, stream);
}

int32_t kvdec_append_attend_cross(kvdec_cache* c, const kvdec_cache* x, const int32_t* lens_host,
                                  const void* k_new, const void* v_new, const float* q_self,
                                  const float* q_cross, int32_t n_q_heads, float scale,
                                  int32_t chunk_self, int32_t chunk_cross, float* out_self,
                                  float* out_cross, void* ws, size_t ws_bytes, void* stream)
{
    g_err.clear();
    // the token's positions: the host mirror, or given (then also set)
    std::vector<int32_t> pre;
    const bool set_device = lens_host != nullptr;
    int32_t rc = set_device ? check_positions(c, lens_host, k_new, v_new, pre)
                            : check_append(c, k_new, v_new);
    if (rc) return rc;
    if (!set_device) pre = c->lens;
    if (!x) return fail(KVDEC_E_INVALID, "cross cache handle is NULL");
    if (!x->d.is_static) return fail(KVDEC_E_STATIC, "the cross part needs a static (encoder) cache");
    rc = check_mirror(x);
    if (rc) return rc;
    if (x->d.batch != c->d.batch || x->d.n_kv_heads != c->d.n_kv_heads || x->d.dtype != c->d.dtype)
        return fail(KVDEC_E_SHAPE, "self and cross caches differ in batch (%d, %d), KV heads (%d, %d) "
                    "or dtype (%d, %d)", c->d.batch, x->d.batch, c->d.n_kv_heads, x->d.n_kv_heads,
                    c->d.dtype, x->d.dtype);
    AttendView sv = view_of(c);
    for (size_t b = 0; b < pre.size(); ++b) {        // rows attended after the append
        const int64_t n = static_cast<int64_t>(pre[b]) + 1;
        sv.rows[b] = static_cast<int32_t>(c->d.window > 0 && n > c->d.window ? c->d.window : n);
    }
    const AttendView xv = view_of(x);
    rc = check_attend(sv, q_self, n_q_heads, scale, chunk_self, out_self, ws, ws_bytes);
    if (rc) return rc;
    rc = check_attend(xv, q_cross, n_q_heads, scale, chunk_cross, out_cross, ws, ws_bytes);
    if (rc) return rc;
    // one workspace holds both parts' partials
    const kvdec::PartialLayout part =
        kvdec::partial_layout(sv.max_chunks + xv.max_chunks, n_q_heads, c->d.batch);
    if (ws_bytes < part.bytes)
        return fail(KVDEC_E_WORKSPACE, "workspace needs %zu bytes for both parts (the sum of the two "
                    "caches' kvdec_workspace_bytes is enough), got %zu", part.bytes, ws_bytes);
    const int32_t group = n_q_heads / c->d.n_kv_heads;
    kvdec::AttendArgs a, xa;
    plan_chunks(sv, group, chunk_self, a);
    plan_chunks(xv, group, chunk_cross, xa);
    auto waves = [&](const kvdec::AttendArgs& p) {
        return kvdec::attend_waves(c->d.dtype, group, p.chunk_rows, p.replay);
    };
    // An automatic chunk size gives way where the parts would need
    // workgroups of different shapes: the automatic part drops to the
    // largest chunk below 256 rows (4-wave workgroups).
    for (int side = 0; side < 2 && waves(a) != waves(xa); ++side) {
        const bool cross_side = side == 0;
        if ((cross_side ? chunk_cross : chunk_self) != 0) continue;
        kvdec::AttendArgs& p = cross_side ? xa : a;
        if (waves(p) > 4 && p.chunk_rows >= 256)
            plan_chunks(cross_side ? xv : sv, group, 192, p);
    }
    if (waves(a) != waves(xa)) {
        // the two parts run on workgroups of different shapes at these chunk
        // sizes: the two calls, in order (same results)
        rc = append_attend_from(c, pre, set_device, k_new, v_new, q_self, n_q_heads, scale,
                                chunk_self, out_self, ws, ws_bytes, stream);
        if (rc) return rc;
        return attend_view(xv, q_cross, n_q_heads, scale, chunk_cross, out_cross, ws, ws_bytes,
                           stream);
    }
    if (c->d.batch > KVDEC_MAX_FUSED_BATCH || c->replay_chunk > 0) {
        // lengths read from (and bumped on) the device
        if (set_device) {
            const hipError_t e = kvdec::launch_set_lens(c->d.lens, pre.data(), c->d.batch,
                                                        static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "set lengths");
            c->lens = pre;             // mirror and device agree even if the attend launch fails
            c->lens_known = true;
        }
        sv.fused_device = true;
    } else {
        sv.fused_lens = pre.data();    // pre-append lengths by value; the launch writes the lengths
    }
    sv.k_new = k_new;
    sv.v_new = v_new;
    sv.lens_out = c->d.lens;
    sv.window = c->d.window;
    fill_args(sv, q_self, scale, out_self, ws, part, a);
    a.x_blocks = xa.n_chunks;
    a.x_q = q_cross;
    a.x_k = x->d.k;
    a.x_v = x->d.v;
    a.x_lens = x->d.lens;
    a.x_out = out_cross;
    a.x_cap_pad = x->cap_pad;
    a.x_row_limit = xa.row_limit;
    a.x_chunk_rows = xa.chunk_rows;
    a.x_one_chunk = xa.one_chunk;
    a.x_uniform = xa.uniform;
    a.need_merge = a.need_merge || xa.need_merge;
    kvdec::MergePlanHost mp;
    if (c->replay_chunk == 0 && x->replay_chunk == 0 && !sv.fused_device && a.need_merge &&
        plan_merge(xv.rows, xa.chunk_rows, 0, true, mp) &&
        plan_merge(sv.rows, a.chunk_rows, xa.n_chunks, false, mp))
        a.merge_plan = &mp;
    const hipError_t e = kvdec::launch_attend(c->d.dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    c->lens = pre;
    for (auto& l : c->lens) ++l;
    if (set_device) c->lens_known = true;     // the positions came from the caller
    return KVDEC_OK;
}

int32_t kvdec_append_attend_noalloc(kvdec_cache* c, const void* k_new, const void* v_new,
                                    const float* q, int32_t n_q_heads, float scale,
                                    int32_t chunk_rows, float* out, void* stream)
{
    g_err.clear();
    const int32_t rc = check_append(c, k_new, v_new);
    if (rc) return rc;
    const std::vector<int32_t> pre = c->lens;
    return append_attend_from(c, pre, false, k_new, v_new, q, n_q_heads, scale, chunk_rows, out,
                              nullptr, 0, stream, true);
}

int32_t kvdec_append_attend_at(kvdec_cache* c, const int32_t* lens_host, const void* k_new,
                               const void* v_new, const float* q, int32_t n_q_heads, float scale,
                               int32_t chunk_rows, float* out, void* ws, size_t ws_bytes,
                               void* stream)
{
    g_err.clear();
    std::vector<int32_t> pre;
    const int32_t rc = check_positions(c, lens_host, k_new, v_new, pre);
    if (rc) return rc;
    return append_attend_from(c, pre, true, k_new, v_new, q, n_q_heads, scale, chunk_rows, out, ws,
                              ws_bytes, stream);
}

const char* kvdec_status_str(int32_t s)
{
    switch (s) {
        case KVDEC_OK: return "ok";
        case KVDEC_E_INVALID: return "invalid argument";
        case KVDEC_E_SHAPE: return "shape error";
        case KVDEC_E_OVERFLOW: return "cache overflow";
        case KVDEC_E_STATIC: return "static/dynamic cache mismatch";
        case KVDEC_E_WORKSPACE: return "workspace too small";
        case KVDEC_E_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* kvdec_last_error(void) { return g_err.c_str(); }

}  // extern "C"
