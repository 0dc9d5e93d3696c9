// Internal interface between the host C-ABI layer (kvdec_api.cpp) and the
// gfx950 kernels (kvdec_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kvdec {

constexpr int kHeadDim = 64;
constexpr int kLensPerLaunch = 256;   // lengths carried by value in one set-lens launch

struct LensBlock {
    int32_t v[kLensPerLaunch];
};

// Workspace of the split-sequence attention: partial results per
// (chunk, query head): unnormalised o[64] and (m, l) with m in log2 units.
struct PartialLayout {
    size_t o_offset;        // float [slots][64]
    size_t ml_offset;       // float2 [slots]
    size_t snap_offset;     // int32 [batch]: pre-append lengths (device-fused append)
    size_t bytes;
};

PartialLayout partial_layout(int64_t max_chunks, int32_t n_q_heads, int32_t batch);

// The merge launch planned on the host (outside replay mode, where the host
// holds every sequence's length): one entry per sequence split over several
// chunks, by value.
constexpr int kMaxMergeEntries = 160;

struct MergePlan {
    int32_t first[kMaxMergeEntries];   // workspace slot of the sequence's first chunk
    int32_t b[kMaxMergeEntries];       // sequence
    int32_t nch[kMaxMergeEntries];     // chunk count; bit 24 set: the cross part's output
};

struct MergePlanHost {
    MergePlan plan;
    int n = 0;
};

// Placement of the chunks of a one-round host-fused launch of the MFMA
// kernel (bf16 K/V, grouped query heads; contiguous or paged cache) on the
// device's compute units.
// The hardware hands the workgroups of a launch that fits one residency
// round out in order of their linear id, round robin over the XCDs and then
// over each XCD's CUs, so ids that agree modulo the CU count run on one CU.  With the grid laid out (KV head, position), a position's
// heads cover n_kv_heads consecutive ids, and positions that agree modulo
// cus / n_kv_heads share their CUs: the host puts the chunks into those
// position classes so that every CU gets about the same rows (largest
// first, each into the least-loaded class).  pos[p] describes the chunk at
// position p (place_entry), kNoChunk an empty position: its sequence, its
// index in the sequence, the sequence's chunk count and its partial slot,
// so a placed workgroup finds its rows without reading the lengths through
// the vector memory path (where its request would queue behind the tile
// loads of the workgroups that started before it on the same CU).  Results
// do not depend on the placement: a chunk's arithmetic and its partial
// slot are the same wherever it runs.
constexpr int kMaxPlaced = 256;
constexpr uint32_t kNoChunk = 0xFFFFFFFFu;

// sequence b < 512, chunk c < 128 of nch < 256, partial slot < 256
constexpr uint32_t place_entry(uint32_t b, uint32_t c, uint32_t nch, uint32_t slot)
{
    return b | (c << 9) | (nch << 16) | (slot << 24);
}

struct Placement {
    uint32_t pos[kMaxPlaced];
    int32_t n = 0;              // positions (0: the grid is (chunk, KV head) in chunk order)
};

struct AttendArgs {
    const float* q;
    const void* k;
    const void* v;
    const int32_t* lens;
    int32_t batch;
    int32_t n_kv_heads;
    int32_t group;          // query heads per KV head
    int32_t cap_pad;        // padded rows per (sequence, KV head): the row stride
    int32_t row_limit;      // rows attended are min(len, row_limit)
    int32_t chunk_rows;     // rows per split-sequence chunk
    int64_t n_chunks;       // sum over sequences of max(1, ceil(len / chunk_rows))
    bool need_merge;        // some sequence spans more than one chunk
    int32_t one_chunk = 0;  // 1: every sequence has exactly one chunk, whatever the
                            // device lengths (grid index = sequence)
    int32_t uniform = -1;   // >= 0: every sequence attends this many rows, known on the
                            // host (the launch reads no length to find its chunk)
    bool replay = false;    // capacity-sized grid (replay mode): surplus workgroups exit at once
    float qscale;           // scale * log2(e)
    float* out;
    void* ws;
    PartialLayout part;
    // paged layout (table == nullptr: contiguous [B][Hkv][cap_pad][64])
    const int32_t* table = nullptr;
    int32_t table_stride = 0;
    int32_t pshift = 0;
    int32_t num_pages = 0;      // pages in the pool (head-major pool)
    // paged fused append (with table and fused_lens): the page each sequence's
    // new row starts, -1 where its page is already in the table
    const int32_t* fresh_pages = nullptr;
    // append fused into the launch (fused_lens != nullptr): pre-append
    // lengths (host), new rows, the device lengths to bump, ring window
    const int32_t* fused_lens = nullptr;
    bool fused_device = false;    // append fused, lengths from the device (merge bumps)
    const void* k_new = nullptr;
    const void* v_new = nullptr;
    int32_t* lens_out = nullptr;
    int32_t window = 0;
    // cross-attention part of a one-launch decoder layer step (x_blocks > 0;
    // contiguous caches, fused append modes only): a static cache attended in
    // the same grid, whose x_blocks workgroups come first along x and whose
    // partials take the first x_blocks slots of the workspace
    int64_t x_blocks = 0;
    const float* x_q = nullptr;
    const void* x_k = nullptr;
    const void* x_v = nullptr;
    const int32_t* x_lens = nullptr;
    float* x_out = nullptr;
    int32_t x_cap_pad = 0;
    int32_t x_row_limit = 0;
    int32_t x_chunk_rows = 0;
    int32_t x_one_chunk = 0;
    int32_t x_uniform = -1;
    // the merge planned on the host (nullptr: the merge finds the chunks
    // from the lengths on the device)
    const MergePlanHost* merge_plan = nullptr;
    // host-fused launches of the MFMA kernel only: the chunks' placement on
    // the CUs (nullptr or n == 0: chunk order)
    const Placement* placement = nullptr;
};

constexpr int kPagesPerLaunch = 256;   // new-page ids carried by value in one paged append

struct PageBlock {
    int32_t v[kPagesPerLaunch];        // new page for each sequence of the slice, or -1
};

constexpr int kEntriesPerLaunch = 256; // block-table entries written by one table-write launch

struct EntryBlock {
    int32_t idx[kEntriesPerLaunch];    // flat index b * table_stride + page slot
    int32_t val[kEntriesPerLaunch];    // page id, or -1
};

hipError_t launch_set_lens(int32_t* lens, const int32_t* host, int32_t n, hipStream_t s);
hipError_t launch_append(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                         int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                         int32_t cap_pad, int32_t window, hipStream_t s);
hipError_t launch_append_slide(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                               int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                               int32_t cap_pad, int32_t keep, hipStream_t s);
hipError_t launch_append_rope(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                              int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                              int32_t cap_pad, int32_t window, const float* q, float* q_rot,
                              int32_t n_q_heads, double theta, hipStream_t s);
hipError_t launch_paged_append(int dtype, void* k_pages, void* v_pages, const void* k_new,
                               const void* v_new, int32_t* lens, int32_t* table,
                               int32_t table_stride, int32_t batch, int32_t n_kv_heads,
                               int32_t pshift, int32_t num_pages, const int32_t* new_pages,
                               bool from_table, hipStream_t s);
hipError_t launch_paged_reserve(int32_t* table, int32_t table_stride, int32_t* lens, int32_t seq,
                                const int32_t* pages, int32_t n_pages, int32_t len, hipStream_t s);
hipError_t launch_table_write(int32_t* table, const int32_t* idx, const int32_t* val, int32_t n,
                              hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_table_clear_tail(int32_t* table, int32_t table_stride, const int32_t* held,
                                   int32_t batch, hipStream_t s);
hipError_t launch_seed(int dtype, void* k, void* v, const void* k_tok, const void* v_tok,
                       int32_t batch, int32_t rows, int32_t n_kv_heads, int32_t cap_pad,
                       hipStream_t s);
hipError_t launch_attend(int dtype, const AttendArgs& a, hipStream_t s);

// Address of the library's device scratch on the current device (looked up
// on the first call per device) and its size.  Used only by the entry point
// that allocates nothing.
hipError_t scratch_device_ptr(void** ptr, size_t* bytes);

// Waves per workgroup the attend kernel for (dtype, group) runs with at this
// chunk size (in capacity-sized replay grids when `replay`): a function of
// these arguments only.  Both parts of a one-launch layer step must agree.
int attend_waves(int dtype, int group, int chunk_rows, bool replay);

// Workgroups of the attend kernel for (dtype, group) that are resident on the
// current device at once (occupancy x compute units); 0 if unknown.  Cached.
int resident_attend_blocks(int dtype, int group);

// Compute units of the current device (0 if unknown); cached per device.
int device_cus();

}  // namespace kvdec
