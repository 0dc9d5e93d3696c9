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

// Workgroups of the attend kernel for (dtype, group) that are resident on the
// current device at once (occupancy x compute units); 0 if unknown.  Cached.
int resident_attend_blocks(int dtype, int group);

}  // namespace kvdec
