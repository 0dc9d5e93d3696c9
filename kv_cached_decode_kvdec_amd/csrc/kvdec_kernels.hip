// gfx950 kernels of the single-token KV-cached decode step.
//
//   append  : scatter one new K/V row per (sequence, KV head) to row lens[b]
//             of the head-major cache, then lens[b] += 1 (pure byte copy);
//             also fused into the attend launch (the workgroup whose chunk
//             holds the new row stores it), and a RoPE form that rotates
//             the key on the way.
//   paged   : the same append through a block table into a head-major page
//             pool, plus the small table writes of the host page allocator.
//   seed    : token-major [B][rows][H*64] -> head-major [B][H][cap][64].
//   attend  : split-sequence decode attention.  One workgroup owns one
//             (sequence, chunk of rows, KV head) and all query heads that
//             share that KV head, so every K/V byte is read from HBM once.
//             Each 16-byte lane load covers 4 f32 / 8 bf16 dims of a row; a
//             row's dot product is finished with DPP butterflies inside the
//             16-lane (f32) or 8-lane (bf16) row group; softmax is online
//             per row slot with exp2 (scale * log2 e applied to each
//             score).  bf16 K/V with 2..8 query heads per KV head runs on
//             MFMA instead (scores and P.V as 16x16x32 bf16 products, q and
//             P split into bf16 hi + lo parts).  A sequence that fits one
//             chunk is finished in place; otherwise each workgroup stores
//             its partial (m, l, o[64]).
//   merge   : log-sum-exp merge of the chunk partials of every
//             (sequence, query head) whose length spans more than one chunk
//             (a second launch, only when some sequence has several chunks.
//             A last-workgroup merge inside the attend kernel needs a
//             device-scope hand-off per workgroup: with a release fence it
//             writes back the XCD's L2 each time; with device-scope stores
//             and a counter it holds every workgroup through a store wait
//             and an atomic round trip, and needs counters that start at
//             zero.  Both cost more than the launch on large grids.)
//
// Arithmetic follows the per-head decode of franken_ocr 0.8.0
// decoder_qwen2.rs (`decode_attn_head`: scores scaled by 1/sqrt(d), max-shifted
// softmax, weighted V sum) with the online-softmax rescaling named in
// whisper-apr 0.3.3 decoder_generated.rs (`compute_attention_cached_with_scratch`,
// Milakov & Gimelshein 2018), and the fail-closed rule of lattice-inference
// 0.4.0 cpu_q8.rs (`full_attention_step_q8`: a denominator that is not > 0
// gives a zero row).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/kvdec.h"
#include "kvdec_internal.h"

namespace kvdec {

namespace {

constexpr int kMaxFusedBatch = KVDEC_MAX_FUSED_BATCH;
constexpr int kMaxPagedFusedBatch = KVDEC_MAX_PAGED_FUSED_BATCH;
constexpr float kNegBig = -1.0e30f;   // finite "no row seen yet" running max

template <int ESZ>
struct Lay {
    static constexpr int kRowBytes = kHeadDim * ESZ;   // 256 (f32) / 128 (bf16)
    static constexpr int kLPR = kRowBytes / 16;        // lanes per row: 16 / 8
    static constexpr int kEPL = 16 / ESZ;              // elements per lane: 4 / 8
    static constexpr int kRPI = 64 / kLPR;             // rows per wave load: 4 / 8
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// All-reduce (sum) over the LPR lanes that hold one row.  xor-1 and xor-2
// via quad permutes, then the half-row and row mirrors; every lane of the
// group ends with the same bits.
template <int LPR>
__device__ __forceinline__ float row_sum(float x)
{
    x += dpp<0xB1>(x);     // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);     // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);    // row_half_mirror
    if constexpr (LPR == 16) x += dpp<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ float row_max16(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both rounded to
// nearest even by the gfx950 conversion v_cvt_pk_bf16_f32 (x - hi is exact
// in f32).  hi + lo carries 16 significant bits of x.
__device__ __forceinline__ void split_bf16(const f32x8 x, bf16x8& hi, bf16x8& lo)
{
    hi = __builtin_convertvector(x, bf16x8);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), bf16x8);
}

// Max and sum over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane swaps, no LDS round trip: permlane32_swap pairs
// each lane with lane ^ 32, permlane16_swap with lane ^ 16.  Every lane ends
// with the same bits (the operations are commutative).
__device__ __forceinline__ float max_over_groups(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The values of lane l and lane l ^ 8 / 16 / 32, ordered (lower lane, upper
// lane), so both lanes of a pair see the same two values in the same order:
// xor 8 by a DPP row rotation, xor 16 and 32 by the gfx950 lane swaps.
__device__ __forceinline__ void lane_pair8(float x, int lane, float& x0, float& x1)
{
    const float p = dpp<0x128>(x);     // row_ror:8 -> lane ^ 8 within each row of 16
    const bool up = lane & 8;
    x0 = up ? p : x;
    x1 = up ? x : p;
}

__device__ __forceinline__ void lane_pair16(float x, float& x0, float& x1)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x0 = __uint_as_float(a[0]);
    x1 = __uint_as_float(a[1]);
}

__device__ __forceinline__ void lane_pair32(float x, float& x0, float& x1)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x0 = __uint_as_float(a[0]);
    x1 = __uint_as_float(a[1]);
}

__device__ __forceinline__ int wave_sum_int(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);   // row_mirror
    const auto a = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    x = static_cast<int>(a[0] + a[1]);
    const auto c = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return static_cast<int>(c[0] + c[1]);
}

__device__ __forceinline__ float sum_over_groups(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// float -> bfloat16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int ESZ>
__device__ __forceinline__ void unpack(const uint4 w, float (&f)[Lay<ESZ>::kEPL])
{
    if constexpr (ESZ == 4) {
        f[0] = __uint_as_float(w.x);
        f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z);
        f[3] = __uint_as_float(w.w);
    } else {
        // bf16 -> f32 is exact: the 16 bits become the high half.
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(u[k] << 16);
            f[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
        }
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// K/V rows are read exactly once per call: nontemporal 16-byte loads keep
// them from displacing useful lines in L2 (measured on MI355X: a plain
// streaming read reaches ~6.1 TB/s, ~7.0 TB/s with nontemporal loads).
__device__ __forceinline__ uint4 load16_stream(const char* p)
{
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Map a flattened chunk index to its sequence.  Chunks are numbered
// sequence by sequence: sequence b owns max(1, ceil(lens[b] / T))
// consecutive indices starting at the exclusive prefix sum (an empty
// sequence keeps one chunk with no rows, which writes its zero row).  Done by one wave with a
// 64-wide scan per group of 64 sequences; all lanes return the same values.
// When the host knows that every sequence has exactly one chunk (one_chunk:
// outside replay mode the grid was sized from the same lengths the kernel
// reads and has B workgroups; in replay mode the row limit fits one chunk),
// chunk blk is sequence blk and no scan is needed.  The grid size alone does
// not tell: a replay grid sized with a horizon can have B workgroups while
// the device lengths have grown past one chunk.
struct Located {
    int b, c, len, nch;
};

// Where an attend launch gets the per-sequence lengths from (LM, the length
// mode):
//  kLensDevice       the device array, rows = lens[b];
//  kLensHostFused    append fused into the launch, the pre-append lengths by
//                    value from the host mirror (the launch reads no device
//                    length), rows = len + 1; the launch bumps the lengths;
//  kLensDeviceFused  append fused into the launch, the pre-append lengths
//                    from the device array (replay mode, any batch), rows =
//                    len + 1; the attend launch snapshots them into the
//                    workspace and the merge launch, which always follows,
//                    reads the snapshot and bumps the lengths (no launch both
//                    reads and writes them).
constexpr int kLensDevice = 0;
constexpr int kLensHostFused = 1;
constexpr int kLensDeviceFused = 2;
constexpr int kLensPagedFused = 3;   // paged cache, append fused, lengths and fresh pages by value

template <int LM>
struct LensSrc;

template <>
struct LensSrc<kLensDevice> {
    const int32_t* lens;
    static constexpr int kPlus = 0;
    __device__ __forceinline__ int get(int b) const { return lens[b]; }
    __device__ __forceinline__ int merge_get(int b) const { return lens[b]; }
    // the length of sequence b0 + lane (0 past the batch), one per lane
    __device__ __forceinline__ int lanes(int b0, int lane, int B) const
    {
        return b0 + lane < B ? lens[b0 + lane] : 0;
    }
};

// the new rows and the cache they are stored into (fused modes)
struct FusedRows {
    const char* k_new;      // [B][Hkv][64] elements
    const char* v_new;
    char* K;                // contiguous cache (or page pools), written at the new row's slot
    char* V;
    int32_t* lens_out;      // device lengths, bumped by one per sequence
    int window;             // ring window, 0 for a linear cache
};

template <>
struct LensSrc<kLensHostFused> {
    int32_t v[kMaxFusedBatch];
    FusedRows f;
    static constexpr int kPlus = 1;
    __device__ __forceinline__ int get(int b) const { return v[b]; }
    __device__ __forceinline__ int merge_get(int b) const { return v[b]; }
    __device__ __forceinline__ int lanes(int b0, int lane, int B) const
    {
        return b0 + lane < B ? v[b0 + lane] : 0;
    }
};

// the paged fused mode: the new rows go to the page pool through the block
// table; a sequence whose new row starts a page brings that page's id
struct PagedFusedRows {
    const char* k_new;      // [B][Hkv][64] elements
    const char* v_new;
    char* K;                // page pools [Hkv][num_pages][page_rows][64]
    char* V;
    int32_t* lens_out;      // device lengths, bumped by one per sequence
    int32_t* table_out;     // device block table, given the fresh pages
};

template <>
struct LensSrc<kLensPagedFused> {
    int32_t v[kMaxPagedFusedBatch];       // pre-append lengths (host mirror)
    int32_t fresh[kMaxPagedFusedBatch];   // page for a row that starts a page, else -1
    PagedFusedRows f;
    static constexpr int kPlus = 1;
    __device__ __forceinline__ int get(int b) const { return v[b]; }
    __device__ __forceinline__ int merge_get(int b) const { return v[b]; }
    __device__ __forceinline__ int lanes(int b0, int lane, int B) const
    {
        return b0 + lane < B ? v[b0 + lane] : 0;
    }
};

template <>
struct LensSrc<kLensDeviceFused> {
    const int32_t* lens;    // pre-append lengths (read by the attend launch only)
    int32_t* snap;          // workspace copy of them (read by the merge launch)
    FusedRows f;
    static constexpr int kPlus = 1;
    __device__ __forceinline__ int get(int b) const { return lens[b]; }
    __device__ __forceinline__ int merge_get(int b) const { return snap[b]; }
    __device__ __forceinline__ int lanes(int b0, int lane, int B) const
    {
        return b0 + lane < B ? lens[b0 + lane] : 0;
    }
};

// Inclusive prefix sum over the 64 lanes of a wave, without LDS: a
// Hillis-Steele scan inside each 16-lane row (DPP row shifts; lanes whose
// source falls off the row add 0), then row 15's total is added to row 1
// and row 3, and lane 31's to rows 2 and 3 (DPP row broadcasts).
__device__ __forceinline__ int wave_inclusive_sum(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
    return x;
}

template <int LM>
__device__ __forceinline__ bool locate(const LensSrc<LM>& ls, int B, int T, int cap, int blk,
                                       int lane, int one_chunk, int uniform, Located& r)
{
    if (uniform >= 0) {
        // every sequence attends `uniform` rows (known on the host): no
        // length is read
        const int nch = max(1, (uniform + T - 1) / T);
        r.b = blk / nch;
        r.c = blk - r.b * nch;
        r.len = uniform;
        r.nch = nch;
        return r.b < B;
    }
    if (one_chunk) {
        const int ln = min(max(ls.get(blk) + LensSrc<LM>::kPlus, 0), cap);
        r.b = blk;
        r.c = 0;
        r.len = __builtin_amdgcn_readfirstlane(ln);
        r.nch = __builtin_amdgcn_readfirstlane(max(1, (ln + T - 1) / T));
        return true;
    }
    int base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bi = b0 + lane;
        const int ln = bi < B ? min(max(ls.lanes(b0, lane, B) + LensSrc<LM>::kPlus, 0), cap) : 0;
        const int cnt = bi < B ? max(1, (ln + T - 1) / T) : 0;
        const int incl = wave_inclusive_sum(cnt);
        // lane values read with readlane are wave-uniform (scalar registers),
        // so the row bounds derived from them stay scalar too
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (blk < base + total) {
            const unsigned long long m = __ballot(incl > blk - base);
            const int first = __ffsll(static_cast<long long>(m)) - 1;
            r.b = b0 + first;
            r.c = blk - base - __builtin_amdgcn_readlane(incl - cnt, first);
            r.len = __builtin_amdgcn_readlane(ln, first);
            r.nch = __builtin_amdgcn_readlane(cnt, first);
            return true;
        }
        base += total;
    }
    return false;
}

// Fused append, inside an attend workgroup of (sequence b, KV head g, chunk c)
// whose rows are [row0, row_end): the workgroup whose rows hold the new
// token's slot stores the new K/V row of head g there, then waits at a
// workgroup barrier, which makes those stores visible to all its waves
// before any of them reads the slot.  No other workgroup reads that slot, so
// the launch needs no wider synchronisation.  Host-fused: the slot's head-0
// workgroup also bumps the length.  Device-fused: workgroup (c 0, head 0)
// snapshots the pre-append length for the merge launch, which bumps it.  (A
// full linear cache puts the slot at row `capacity`, past every chunk: no
// store, and the merge leaves the length as it is.)
template <int RB, int LM>
__device__ __forceinline__ void fused_append(const LensSrc<LM>& ls, const Located& loc, int g,
                                            int Hkv, int cap_pad, int row0, int row_end)
{
    const int b = loc.b;
    const int len0 = ls.get(b);
    const int slot = ls.f.window > 0 ? len0 % ls.f.window : len0;
    if (row0 <= slot && slot < row_end) {
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        constexpr int VPR = RB / 16;
        for (int t = threadIdx.x; t < 2 * VPR; t += blockDim.x) {
            const bool isv = t >= VPR;
            const int w = isv ? t - VPR : t;
            const uint4 x = reinterpret_cast<const uint4*>((isv ? ls.f.v_new : ls.f.k_new) + hg * RB)[w];
            reinterpret_cast<uint4*>((isv ? ls.f.V : ls.f.K) + (hg * cap_pad + slot) * RB)[w] = x;
        }
        if constexpr (LM == kLensHostFused)
            if (g == 0 && threadIdx.x == 0) ls.f.lens_out[b] = len0 + 1;
        __syncthreads();
    }
    if constexpr (LM == kLensDeviceFused)
        if (loc.c == 0 && g == 0 && threadIdx.x == 0) ls.snap[b] = len0;
}

// Fused append into a contiguous cache, inside the attend workgroup of
// (sequence b, KV head g, chunk c) whose rows [row0, row_end) hold the new
// token's slot.  No barrier: every load of this launch that would read the
// slot row reads the new row from k_new / v_new instead (kn / vn, plus the
// lane's byte offset in the row), so no load waits for the row to be stored,
// and threads 0 .. 2 * RB / 16 - 1 copy the row into the cache (store(),
// called once the workgroup's first loads are issued).  No other workgroup
// reads the slot.  Host-fused: the slot's head-0 workgroup also bumps the
// length.  Device-fused: workgroup (c 0, head 0) snapshots the pre-append
// length for the merge launch, which bumps it.  (A full linear cache puts
// the slot at row `capacity`, past every chunk: no copy, and the merge
// leaves the length as it is.)
template <int RB>
struct FreshRow {
    int row = -1;               // the slot, if this chunk holds it (wave-uniform), else -1
    const char* kn;             // the new K / V row (wave-uniform; the cache base while row < 0)
    const char* vn;
    char* dst = nullptr;        // the copying thread's 16 bytes of the slot
    uint4 val{};
    __device__ __forceinline__ FreshRow(const char* K, const char* V) : kn(K), vn(V) {}
    __device__ __forceinline__ void store() const
    {
        if (dst) *reinterpret_cast<uint4*>(dst) = val;
    }
    // the address a load of row r reads: the new row (at byte `piece` of
    // it) for the slot, the cache address otherwise
    __device__ __forceinline__ const char* pick_k(int r, int piece, const char* cache) const
    {
        return r == row ? kn + piece : cache;
    }
    __device__ __forceinline__ const char* pick_v(int r, int piece, const char* cache) const
    {
        return r == row ? vn + piece : cache;
    }
};

template <int RB, int LM>
__device__ __forceinline__ FreshRow<RB> fresh_row(const LensSrc<LM>& ls, const Located& loc, int g,
                                                  int Hkv, int cap_pad, int row0, int row_end)
{
    FreshRow<RB> fr(ls.f.K, ls.f.V);
    const int b = loc.b;
    const int len0 = ls.get(b);
    const int slot = ls.f.window > 0 ? len0 % ls.f.window : len0;
    if (row0 <= slot && slot < row_end) {
        constexpr int VPR = RB / 16;
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        const char* k_new = ls.f.k_new + hg * RB;
        const char* v_new = ls.f.v_new + hg * RB;
        fr.row = slot;
        fr.kn = k_new;
        fr.vn = v_new;
        if (threadIdx.x < 2 * VPR) {
            const bool isv = threadIdx.x >= VPR;
            const int w = isv ? threadIdx.x - VPR : threadIdx.x;
            char* K = ls.f.K;
            char* V = ls.f.V;
            fr.val = *reinterpret_cast<const uint4*>((isv ? v_new : k_new) + 16 * w);
            fr.dst = (isv ? V : K) + (hg * cap_pad + slot) * RB + 16 * w;
        }
        if constexpr (LM == kLensHostFused)
            if (g == 0 && threadIdx.x == 0) ls.f.lens_out[b] = len0 + 1;
    }
    if constexpr (LM == kLensDeviceFused)
        if (loc.c == 0 && g == 0 && threadIdx.x == 0) ls.snap[b] = len0;
    return fr;
}

// Combine the WAVES per-wave states of a workgroup (staged in LDS) and
// write either the normalised output row (sequence fits one chunk) or the
// chunk partial (m, l, o[64]) for the merge launch.
template <int WAVES, int GROUP>
__device__ __forceinline__ void finish_block(const float (&sm_o)[WAVES][GROUP][kHeadDim],
                                             const float (&sm_m)[WAVES][GROUP],
                                             const float (&sm_l)[WAVES][GROUP], int wave, int lane,
                                             const Located& loc, int g, int Hq, int slot_chunk,
                                             float* __restrict__ out, float* __restrict__ part_o,
                                             float2* __restrict__ part_ml)
{
    __syncthreads();
    for (int i = wave; i < GROUP; i += WAVES) {
        float M = sm_m[0][i];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) M = fmaxf(M, sm_m[w][i]);
        float Lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float c = fast_exp2(sm_m[w][i] - M);
            Lsum = fmaf(sm_l[w][i], c, Lsum);
            acc = fmaf(sm_o[w][i][lane], c, acc);
        }
        const int h = g * GROUP + i;
        if (loc.nch == 1) {
            out[(static_cast<size_t>(loc.b) * Hq + h) * kHeadDim + lane] =
                (Lsum > 0.f) ? acc / Lsum : 0.f;
        } else {
            const size_t slot = static_cast<size_t>(slot_chunk) * Hq + h;
            part_o[slot * kHeadDim + lane] = acc;
            if (lane == 0) part_ml[slot] = make_float2(M, Lsum);
        }
    }
}


// Paged layout: row r of (sequence b, KV head g) lives in page
// table[b * table_stride + (r >> pshift)], slot r & (2^pshift - 1).  The pool
// is head-major, [n_kv_heads][num_pages][2^pshift rows][64]: one page id
// covers every KV head, and consecutive page ids of one head are adjacent,
// so a sequence whose pages were taken in order reads each head as one
// stream.  A workgroup stages the page ids of its chunk in LDS once, then
// addresses rows from them.
struct PageMap {
    const int32_t* table;   // device block table (nullptr: contiguous layout)
    int stride;             // entries per sequence
    int pshift;             // log2(rows per page)
    int num_pages;          // pages in the pool
};

constexpr int kMaxChunkPages = KVDEC_MAX_CHUNK / 16 + 1;

// The cross-attention part of a one-launch decoder layer step (self append +
// attend and cross attend in one grid): its workgroups come first along x
// (they read the longer rows: started first, they leave the shorter
// self-attention workgroups to fill the tail); it reads a static cache with
// lengths from the device, has its own chunk size, and writes its own
// output.  Its chunk partials take the first n_blocks slots of the
// workspace, the self part's the slots after them.
struct CrossPart {
    const float* q;         // [B][Hq][64]
    const char* K;          // static cache [B][Hkv][cap_pad][64]
    const char* V;
    const int32_t* lens;    // device lengths of the static cache
    float* out;             // [B][Hq][64]
    int cap_pad;
    int row_limit;
    int T;                  // chunk rows
    int one_chunk;          // every sequence has exactly one chunk
    int uniform;            // rows every sequence attends, when the host knows them; else -1
    int n_blocks;           // chunks of the part (0: no cross part)
};

// Where an attend workgroup sits: its part, KV head, chunk index within the
// part's grid, and the workspace slot of its partials.  Without a cross part
// the grid is (KV heads, chunks) for ragged lengths in a contiguous cache
// and (chunks, KV heads) otherwise: the hardware hands workgroups to the 8
// XCDs by linear id modulo 8, and with the heads innermost each XCD gets
// an equal share of every chunk of ragged lengths (qwen2-0.5b 73.4 -> 72.0
// us per step); equal-length launches and the paged pool (whose heads lie
// far apart) were slower that way (whisper-large as two calls 100.3 ->
// 101.9 us, qwen2-0.5b with 16-row pages 75.7 -> 76.7 us).  With a cross
// part it is one-dimensional, every cross workgroup (all heads) before every
// self workgroup, so that the longer cross work is dispatched first and the
// shorter self work fills the tail: the Whisper-large step takes 96.4 us this way, against 100.8 us
// as two launches, 103.5 us with the parts ordered along x within each head
// (which mixes them through the whole launch) and 111.8 us alternating them
// block by block.  Within the cross part the KV head runs fastest: every
// sequence has the same encoder length and so the same chunk sizes, and
// with chunks innermost a chunk count that is a multiple of the 8 XCDs
// (workgroup id modulo 8) would send every head's copy of one chunk index,
// the short last chunk included, to one XCD (Whisper-base: 12 chunks of
// 128 rows, 21.5 against 20.2 us per step).  The self part keeps chunks
// innermost (with heads innermost the Whisper-large step lost 0.5 us).
struct BlockPos {
    bool in_cross;
    int g;          // KV head
    int blk;        // chunk index within the part
    int slot;       // workspace slot index: cross chunks first, then self chunks
};

template <bool X2>
__device__ __forceinline__ BlockPos block_pos(const CrossPart& xp, int Hkv, int uniform)
{
    BlockPos p;
    if constexpr (X2) {
        const int L = static_cast<int>(blockIdx.x);
        const int nxh = xp.n_blocks * Hkv;
        p.in_cross = L < nxh;
        const int Lp = p.in_cross ? L : L - nxh;
        if (p.in_cross) {
            p.blk = Lp / Hkv;
            p.g = Lp - p.blk * Hkv;
        } else {
            const int nb = (static_cast<int>(gridDim.x) - nxh) / Hkv;
            p.g = Lp / nb;
            p.blk = Lp - p.g * nb;
        }
        p.slot = p.in_cross ? p.blk : xp.n_blocks + p.blk;
    } else {
        p.in_cross = false;
        // (the launch keeps chunks along x where they would pass the 65535
        // limit of the y dimension; gridDim.x then exceeds any head count)
        const bool heads_x = uniform < 0 && static_cast<int>(gridDim.x) == Hkv;
        p.g = static_cast<int>(heads_x ? blockIdx.x : blockIdx.y);
        p.blk = static_cast<int>(heads_x ? blockIdx.y : blockIdx.x);
        p.slot = p.blk;
    }
    return p;
}

// A host-fused launch of the MFMA kernel (contiguous or paged) with a
// placement runs on a (KV head, position) grid: the workgroup takes the chunk the host put at
// its position, with its sequence, index and chunk count from the entry and
// the sequence's length from the by-value lengths (scalar reads only).
// Returns 1 with loc filled, 0 where the launch has no placement (locate
// finds the chunk), -1 for an empty position (nothing to do).
template <int LM, bool X2>
__device__ __forceinline__ int placed(const Placement& pl, const LensSrc<LM>& ls, int cap,
                                      BlockPos& p, Located& loc)
{
    if constexpr ((LM == kLensHostFused || LM == kLensPagedFused) && !X2) {
        if (pl.n > 0) {
            const uint32_t e = pl.pos[blockIdx.y];
            if (e == kNoChunk) return -1;
            p.g = static_cast<int>(blockIdx.x);
            p.blk = static_cast<int>(e >> 24);
            p.slot = p.blk;
            loc.b = static_cast<int>(e & 511u);
            loc.c = static_cast<int>((e >> 9) & 127u);
            loc.nch = static_cast<int>((e >> 16) & 255u);
            loc.len = min(max(ls.v[loc.b] + LensSrc<LM>::kPlus, 0), cap);
            return 1;
        }
    }
    return 0;
}

// fresh_idx >= 0: table entry fresh_idx is being given page fresh_page by this
// launch (the paged fused append); it is taken from there, not read.
template <bool PAGED>
__device__ __forceinline__ void stage_pages(const PageMap& pm, int b, int row0, int row_end,
                                            int* sm_pages, int fresh_idx = -1, int fresh_page = -1)
{
    if constexpr (PAGED) {
        const int p0 = row0 >> pm.pshift;
        const int np = row_end > row0 ? ((row_end - 1) >> pm.pshift) - p0 + 1 : 0;
        for (int t = threadIdx.x; t < np; t += blockDim.x)
            sm_pages[t] = p0 + t == fresh_idx ? fresh_page
                                              : pm.table[static_cast<size_t>(b) * pm.stride + p0 + t];
        __syncthreads();
    }
}

// Paged fused append, in the attend workgroup of (sequence b, KV head g,
// chunk c) that holds the new row's slot: store the new K/V row of head g at
// its pool row, give the block table the fresh page (head 0), bump the
// length (head 0), then a workgroup barrier before any wave reads the slot.
// A fresh page starts at the new row, so no other chunk of the sequence
// covers it, and every workgroup of this chunk took it from the arguments.
template <int RB>
__device__ __forceinline__ void fused_append_paged(const LensSrc<kLensPagedFused>& ls,
                                                  const Located& loc, int g, int Hkv,
                                                  const PageMap& pm, const int* sm_pages, int row0,
                                                  int row_end)
{
    const int b = loc.b;
    const int len0 = ls.v[b];
    if (row0 <= len0 && len0 < row_end) {
        const int page = sm_pages[(len0 >> pm.pshift) - (row0 >> pm.pshift)];
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        const size_t row = ((static_cast<size_t>(g) * pm.num_pages + page) << pm.pshift) +
                           (len0 & ((1 << pm.pshift) - 1));
        constexpr int VPR = RB / 16;
        if (threadIdx.x < VPR)
            reinterpret_cast<uint4*>(ls.f.K + row * RB)[threadIdx.x] =
                reinterpret_cast<const uint4*>(ls.f.k_new + hg * RB)[threadIdx.x];
        else if (threadIdx.x < 2 * VPR)
            reinterpret_cast<uint4*>(ls.f.V + row * RB)[threadIdx.x - VPR] =
                reinterpret_cast<const uint4*>(ls.f.v_new + hg * RB)[threadIdx.x - VPR];
        if (g == 0 && threadIdx.x == 0) {
            if (ls.fresh[b] >= 0)
                ls.f.table_out[static_cast<size_t>(b) * pm.stride + (len0 >> pm.pshift)] = ls.fresh[b];
            ls.f.lens_out[b] = len0 + 1;
        }
        __syncthreads();
    }
}

// Paged cache, device-fused mode (replay): the new row's page comes from the
// block table, where the host put it before the replay; the workgroup whose
// chunk holds the slot stores the row there, then a workgroup barrier.  A
// slot whose table entry holds no page is neither stored nor attended (the
// chunk ends before it; the merge launch then leaves the length as it is).
// Workgroup (chunk 0, head 0) snapshots the pre-append length for the merge.
template <int RB>
__device__ __forceinline__ void fused_append_paged_device(const LensSrc<kLensDeviceFused>& ls,
                                                         const Located& loc, int g, int Hkv,
                                                         const PageMap& pm, const int* sm_pages,
                                                         int row0, int& row_end)
{
    const int b = loc.b;
    const int len0 = ls.get(b);
    if (row0 <= len0 && len0 < row_end) {
        const int page = sm_pages[(len0 >> pm.pshift) - (row0 >> pm.pshift)];
        if (page < 0 || page >= pm.num_pages) {
            row_end = len0;
        } else {
            const size_t hg = static_cast<size_t>(b) * Hkv + g;
            const size_t row = ((static_cast<size_t>(g) * pm.num_pages + page) << pm.pshift) +
                               (len0 & ((1 << pm.pshift) - 1));
            constexpr int VPR = RB / 16;
            if (threadIdx.x < VPR)
                reinterpret_cast<uint4*>(ls.f.K + row * RB)[threadIdx.x] =
                    reinterpret_cast<const uint4*>(ls.f.k_new + hg * RB)[threadIdx.x];
            else if (threadIdx.x < 2 * VPR)
                reinterpret_cast<uint4*>(ls.f.V + row * RB)[threadIdx.x - VPR] =
                    reinterpret_cast<const uint4*>(ls.f.v_new + hg * RB)[threadIdx.x - VPR];
            __syncthreads();
        }
    }
    if (loc.c == 0 && g == 0 && threadIdx.x == 0) ls.snap[b] = len0;
}

// Byte offset of row r of (sequence b, KV head g) from the pool / cache base.
template <bool PAGED, int RB>
__device__ __forceinline__ size_t row_offset(const PageMap& pm, const int* sm_pages, int b, int g,
                                             int Hkv, int cap_pad, int row0, int r)
{
    if constexpr (PAGED) {
        const int page = sm_pages[(r >> pm.pshift) - (row0 >> pm.pshift)];
        const size_t rows = ((static_cast<size_t>(g) * pm.num_pages + page) << pm.pshift) +
                            (r & ((1 << pm.pshift) - 1));
        return rows * RB;
    } else {
        return ((static_cast<size_t>(b) * Hkv + g) * cap_pad + r) * RB;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// set lengths (values carried by value; no host-to-device copy)
// ---------------------------------------------------------------------------
__global__ void set_lens_kernel(int32_t* __restrict__ lens, int32_t n, LensBlock vals)
{
    const int t = threadIdx.x;
    if (t < n) lens[t] = vals.v[t];
}

// ---------------------------------------------------------------------------
// append: one workgroup per sequence; 16-byte copies; the length is bumped
// after the workgroup barrier so no thread reads the new value.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__global__ __launch_bounds__(256) void append_kernel(char* __restrict__ K, char* __restrict__ V,
                                                     const char* __restrict__ kn,
                                                     const char* __restrict__ vn,
                                                     int32_t* __restrict__ lens, int Hkv,
                                                     int capacity, int cap_pad, int window)
{
    constexpr int VPR = ROW_BYTES / 16;
    const int b = blockIdx.x;
    const int len = lens[b];
    // linear cache: row `len`, refused at capacity (the host already rejected
    // it); sliding-window ring: slot len % window, the oldest row is replaced
    if (len < 0 || len == INT32_MAX || (window == 0 && len >= capacity)) return;
    const int slot = window > 0 ? len % window : len;
    const int n = Hkv * VPR;
    for (int t = threadIdx.x; t < 2 * n; t += blockDim.x) {
        const bool isv = t >= n;
        const int tt = isv ? t - n : t;
        const int g = tt / VPR, w = tt - g * VPR;
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        const uint4* src = reinterpret_cast<const uint4*>((isv ? vn : kn) + hg * ROW_BYTES) + w;
        uint4* dst = reinterpret_cast<uint4*>((isv ? V : K) +
                                              (hg * cap_pad + slot) * ROW_BYTES) + w;
        *dst = *src;
    }
    __syncthreads();
    if (threadIdx.x == 0) lens[b] = len + 1;
}

// ---------------------------------------------------------------------------
// append with a sliding window that keeps an overlap (the streaming cache of
// whisper-apr 0.3.3 decoder_generated.rs, `StreamingKVCache`): a sequence
// whose new row would pass the capacity first keeps only its last `keep`
// rows, moved to rows 0 .. keep - 1 (keep <= capacity / 2, so the source rows
// capacity - keep .. capacity - 1 and the destination rows never overlap),
// and restarts at length `keep`; then the row is appended.  The decision is
// taken on the device from the length there, so it also holds in replay
// mode.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__global__ __launch_bounds__(256) void append_slide_kernel(char* __restrict__ K, char* __restrict__ V,
                                                           const char* __restrict__ kn,
                                                           const char* __restrict__ vn,
                                                           int32_t* __restrict__ lens, int Hkv,
                                                           int capacity, int cap_pad, int keep)
{
    constexpr int VPR = ROW_BYTES / 16;
    const int b = blockIdx.x;
    int len = lens[b];
    if (len < 0 || len > capacity) return;
    if (len + 1 > capacity) {
        const int from = len - keep;
        const int per_head = keep * VPR;
        const int n = Hkv * per_head;
        for (int t = threadIdx.x; t < 2 * n; t += blockDim.x) {
            const bool isv = t >= n;
            const int tt = isv ? t - n : t;
            const int g = tt / per_head, rem = tt - g * per_head;
            const int r = rem / VPR, w = rem - r * VPR;
            char* base = (isv ? V : K) + (static_cast<size_t>(b) * Hkv + g) * cap_pad * ROW_BYTES;
            reinterpret_cast<uint4*>(base + static_cast<size_t>(r) * ROW_BYTES)[w] =
                reinterpret_cast<const uint4*>(base + static_cast<size_t>(from + r) * ROW_BYTES)[w];
        }
        // every moved row is read before the new row (at row `keep`, which may
        // be the first source row) is written
        __syncthreads();
        len = keep;
    }
    const int n = Hkv * VPR;
    for (int t = threadIdx.x; t < 2 * n; t += blockDim.x) {
        const bool isv = t >= n;
        const int tt = isv ? t - n : t;
        const int g = tt / VPR, w = tt - g * VPR;
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        reinterpret_cast<uint4*>((isv ? V : K) + (hg * cap_pad + len) * ROW_BYTES)[w] =
            reinterpret_cast<const uint4*>((isv ? vn : kn) + hg * ROW_BYTES)[w];
    }
    __syncthreads();
    if (threadIdx.x == 0) lens[b] = len + 1;
}

// ---------------------------------------------------------------------------
// append with rotary position embedding: the new key (and optionally the
// query) of every sequence is rotated at the token's position (= its length
// before the append) before the key is stored -- the RoPE-then-append order
// of franken_ocr 0.8.0 decoder_qwen2.rs (`qwen2_decode_step`), NEOX
// rotate-half pairs (i, i + 32) as in lattice-inference 0.4.0 cpu_q8.rs
// (`full_attention_step_q8`), angle pos * theta^(-2i/64).  Angles, sin/cos
// and the rotation are computed in double (positions reach 8k and beyond,
// where a float angle would be off by ~1e-3 rad); the result is rounded to
// float, then to bf16 (nearest even) for bf16 caches.
// ---------------------------------------------------------------------------
template <int ESZ>
__global__ __launch_bounds__(256) void append_rope_kernel(
    char* __restrict__ K, char* __restrict__ V, const char* __restrict__ kn,
    const char* __restrict__ vn, int32_t* __restrict__ lens, int Hkv, int capacity, int cap_pad,
    int window, const float* q_in, float* q_out, int Hq, double theta)
{
    constexpr int RB = kHeadDim * ESZ;
    constexpr int VPR = RB / 16;
    const int b = blockIdx.x;
    const int len = lens[b];
    if (len < 0 || len == INT32_MAX || (window == 0 && len >= capacity)) return;
    const int slot = window > 0 ? len % window : len;
    const double pos = static_cast<double>(len);
    const int rot_rows = Hkv + (q_in ? Hq : 0);
    for (int t = threadIdx.x; t < rot_rows * 32; t += blockDim.x) {
        const int row = t >> 5, i = t & 31;
        double sn, cs;
        sincos(pos * pow(theta, -2.0 * i / 64.0), &sn, &cs);
        if (row < Hkv) {
            const size_t hg = static_cast<size_t>(b) * Hkv + row;
            double x0, x1;
            if constexpr (ESZ == 4) {
                const float* src = reinterpret_cast<const float*>(kn) + hg * kHeadDim;
                x0 = src[i];
                x1 = src[i + 32];
            } else {
                const uint16_t* src = reinterpret_cast<const uint16_t*>(kn) + hg * kHeadDim;
                x0 = __uint_as_float(static_cast<uint32_t>(src[i]) << 16);
                x1 = __uint_as_float(static_cast<uint32_t>(src[i + 32]) << 16);
            }
            const float y0 = static_cast<float>(x0 * cs - x1 * sn);
            const float y1 = static_cast<float>(x0 * sn + x1 * cs);
            const size_t dst = (hg * cap_pad + slot) * kHeadDim;
            if constexpr (ESZ == 4) {
                reinterpret_cast<float*>(K)[dst + i] = y0;
                reinterpret_cast<float*>(K)[dst + i + 32] = y1;
            } else {
                reinterpret_cast<uint16_t*>(K)[dst + i] = static_cast<uint16_t>(bf16_rne(y0));
                reinterpret_cast<uint16_t*>(K)[dst + i + 32] = static_cast<uint16_t>(bf16_rne(y1));
            }
        } else {
            // q_in and q_out may alias: each thread reads and writes its own pair
            const size_t qi = (static_cast<size_t>(b) * Hq + (row - Hkv)) * kHeadDim;
            const double x0 = q_in[qi + i], x1 = q_in[qi + i + 32];
            q_out[qi + i] = static_cast<float>(x0 * cs - x1 * sn);
            q_out[qi + i + 32] = static_cast<float>(x0 * sn + x1 * cs);
        }
    }
    // V rows: plain 16-byte copies
    for (int t = threadIdx.x; t < Hkv * VPR; t += blockDim.x) {
        const int g = t / VPR, w = t - g * VPR;
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        reinterpret_cast<uint4*>(V + (hg * cap_pad + slot) * RB)[w] =
            reinterpret_cast<const uint4*>(vn + hg * RB)[w];
    }
    __syncthreads();
    if (threadIdx.x == 0) lens[b] = len + 1;
}

// ---------------------------------------------------------------------------
// paged append: a page pool [n_kv_heads][num_pages][2^pshift rows][64] and a
// block table per sequence (the paged cache of whisper-apr 0.3.3
// decoder_generated.rs, `PagedDecoderKVCache`: page = position / page size,
// slot = position % page size).  When a sequence's row lands at the start of
// a page, the host has chosen a free page for it (passed by value); the
// kernel installs it in the table before writing the row.  With from_table
// (replay mode) every row's page comes from the table, where the host put it
// ahead of the replays; a row whose entry holds no page is not written and
// its sequence keeps its length.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__global__ __launch_bounds__(256) void paged_append_kernel(
    char* __restrict__ Kp, char* __restrict__ Vp, const char* __restrict__ kn,
    const char* __restrict__ vn, int32_t* __restrict__ lens, int32_t* __restrict__ table,
    int table_stride, int Hkv, int pshift, int num_pages, int b0, PageBlock new_pages,
    int from_table)
{
    constexpr int VPR = ROW_BYTES / 16;
    const int b = b0 + blockIdx.x;
    const int len = lens[b];
    if (len < 0) return;
    const int pidx = len >> pshift;
    if (pidx >= table_stride) return;                 // full: nothing written
    const int slot = len & ((1 << pshift) - 1);
    int32_t* entry = table + static_cast<size_t>(b) * table_stride + pidx;
    int page;
    if (slot == 0 && !from_table) {
        page = new_pages.v[blockIdx.x];
        if (page < 0) return;                         // host already rejected this
        if (threadIdx.x == 0) *entry = page;
    } else {
        page = *entry;
    }
    if (page < 0 || page >= num_pages) return;        // no page holds this row: nothing written
    const int n = Hkv * VPR;
    for (int t = threadIdx.x; t < 2 * n; t += blockDim.x) {
        const bool isv = t >= n;
        const int tt = isv ? t - n : t;
        const int g = tt / VPR, w = tt - g * VPR;
        const size_t hg = static_cast<size_t>(b) * Hkv + g;
        const size_t row = ((static_cast<size_t>(g) * num_pages + page) << pshift) + slot;
        const uint4* src = reinterpret_cast<const uint4*>((isv ? vn : kn) + hg * ROW_BYTES) + w;
        uint4* dst = reinterpret_cast<uint4*>((isv ? Vp : Kp) + row * ROW_BYTES) + w;
        *dst = *src;
    }
    __syncthreads();
    if (threadIdx.x == 0) lens[b] = len + 1;
}

// Install host-chosen pages in a block table (one sequence, a slice of its
// entries) and set the sequence's length: the prefill hand-off of a paged
// cache, whose rows the caller writes itself.
__global__ void paged_reserve_kernel(int32_t* __restrict__ table, int32_t* __restrict__ lens,
                                     int seq, int first, int n, int len, PageBlock pages)
{
    const int t = threadIdx.x;
    if (t < n) table[first + t] = pages.v[t];
    if (t == 0 && len >= 0) lens[seq] = len;
}

// Fill n int32 values (a new paged cache's block table with -1).
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v)
{
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = v;
}

// Set -1 in every block-table entry past the first held[b] of each sequence
// of a slice (entering replay mode).
__global__ void table_clear_tail_kernel(int32_t* __restrict__ table, int stride, int b0,
                                        LensBlock held)
{
    int32_t* row = table + static_cast<size_t>(b0 + blockIdx.x) * stride;
    for (int i = held.v[blockIdx.x] + threadIdx.x; i < stride; i += blockDim.x) row[i] = -1;
}

// Write block-table entries (flat indices and values carried by value):
// pages given ahead of replays, and -1 where pages return to the pool.
__global__ void table_write_kernel(int32_t* __restrict__ table, int n, EntryBlock e)
{
    const int t = threadIdx.x;
    if (t < n) table[e.idx[t]] = e.val[t];
}

// ---------------------------------------------------------------------------
// seed: token-major -> head-major, grid-stride over 16-byte words.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__global__ __launch_bounds__(256) void seed_kernel(char* __restrict__ K, char* __restrict__ V,
                                                   const char* __restrict__ kt,
                                                   const char* __restrict__ vt, int B, int rows,
                                                   int Hkv, int cap_pad)
{
    constexpr int VPR = ROW_BYTES / 16;
    const size_t n = static_cast<size_t>(B) * rows * Hkv * VPR;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < 2 * n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const bool isv = i >= n;
        size_t j = isv ? i - n : i;
        const int w = static_cast<int>(j % VPR);
        j /= VPR;
        const int g = static_cast<int>(j % Hkv);
        j /= Hkv;
        const int t = static_cast<int>(j % rows);
        const size_t b = j / rows;
        const uint4* src = reinterpret_cast<const uint4*>(isv ? vt : kt) +
                           ((b * rows + t) * Hkv + g) * VPR + w;
        uint4* dst = reinterpret_cast<uint4*>(isv ? V : K) +
                     ((b * Hkv + g) * cap_pad + t) * VPR + w;
        *dst = *src;
    }
}

// ---------------------------------------------------------------------------
// attend
// ---------------------------------------------------------------------------
// Lane layout inside a wave: lane = sub * LPR + part.  `part` selects 16
// bytes (EPL dims) of a row, `sub` the row slot (RPI slots per load).  One
// wave iteration loads U rows per slot: rows r0 + u * RPI + sub.
// WAVES waves interleave over the chunk in steps of U * RPI rows.
// Waves per SIMD the VALU kernel asks the compiler to fit (1: no request):
// f32 groups 2 and 6 land one or two VGPRs past an occupancy step without it.
template <int ESZ, int GROUP>
constexpr int valu_min_waves() { return ESZ == 4 && GROUP == 2 ? 7 : ESZ == 4 && GROUP == 6 ? 4 : ESZ == 2 && GROUP == 1 ? 7 : 1; }

template <int ESZ, int GROUP, int WAVES, int U, bool PAGED, int LM, bool X2>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(valu_min_waves<ESZ, GROUP>())))
void attend_kernel(
    const float* __restrict__ q, const char* __restrict__ K, const char* __restrict__ V,
    LensSrc<LM> ls, int B, int Hkv, int cap_pad, int row_limit, int T, int one_chunk, int uniform,
    float qscale, float* __restrict__ out, float* __restrict__ part_o, float2* __restrict__ part_ml,
    PageMap pm, CrossPart xp)
{
    static_assert(!(X2 && PAGED), "the one-launch layer step reads contiguous caches");
    using L = Lay<ESZ>;
    constexpr int EPL = L::kEPL, LPR = L::kLPR, RPI = L::kRPI, RB = L::kRowBytes;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;
    const int part = lane - sub * LPR;
    const BlockPos pos = block_pos<X2>(xp, Hkv, PAGED ? 0 : uniform);
    const int g = pos.g;
    const int Hq = Hkv * GROUP;

    Located loc;
    const bool in_cross = pos.in_cross;     // workgroup-uniform
    if (in_cross) {
        const LensSrc<kLensDevice> xs{xp.lens};
        if (!locate<kLensDevice>(xs, B, xp.T, xp.row_limit, pos.blk, lane, xp.one_chunk, xp.uniform,
                                 loc))
            return;
        q = xp.q;
        K = xp.K;
        V = xp.V;
        out = xp.out;
        cap_pad = xp.cap_pad;
        T = xp.T;
    } else {
        if (!locate<LM>(ls, B, T, row_limit, pos.blk, lane, one_chunk, uniform, loc)) return;
    }
    const int row0 = loc.c * T;
    int row_end = min(loc.len, row0 + T);   // lowered where a replayed row has no page

    __shared__ int sm_pages[PAGED ? kMaxChunkPages : 1];
    if constexpr (LM == kLensPagedFused)
        stage_pages<PAGED>(pm, loc.b, row0, row_end, sm_pages,
                           ls.fresh[loc.b] >= 0 ? (ls.v[loc.b] >> pm.pshift) : -1, ls.fresh[loc.b]);
    else
        stage_pages<PAGED>(pm, loc.b, row0, row_end, sm_pages);
    const char* Kb = K + part * 16;
    const char* Vb = V + part * 16;
    if constexpr (LM == kLensPagedFused)
        fused_append_paged<RB>(ls, loc, g, Hkv, pm, sm_pages, row0, row_end);
    else if constexpr (PAGED && LM == kLensDeviceFused)
        fused_append_paged_device<RB>(ls, loc, g, Hkv, pm, sm_pages, row0, row_end);
    else if constexpr (LM != kLensDevice)
        if (!in_cross) fused_append<RB>(ls, loc, g, Hkv, cap_pad, row0, row_end);

    // q for the GROUP heads sharing KV head g, this lane's dims.  It is not
    // waited for before the loop: the first rows' loads are issued first and
    // the scale (times log2 e) is applied to each score, so the workgroup
    // pays one memory round trip before its first scores, not two.
    float4 qv[GROUP][EPL / 4];
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
        const float* qp = q + (static_cast<size_t>(loc.b) * Hq + g * GROUP + i) * kHeadDim + part * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) qv[i][e / 4] = *reinterpret_cast<const float4*>(qp + e);
    }

    float m[GROUP], l[GROUP], o[GROUP][EPL];
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
        m[i] = kNegBig;
        l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[i][e] = 0.f;
    }

    constexpr int kWaveRows = U * RPI;
    for (int r0 = row0 + wave * kWaveRows; r0 < row_end; r0 += WAVES * kWaveRows) {
        // full: every row of this iteration lies inside the chunk (wave-uniform)
        const bool full = r0 + kWaveRows <= row_end;
        uint4 kr[U], vr[U];
        // rows past the end repeat the last row (weight zero, finite V)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(r0 + u * RPI + sub, row_end - 1);
            const size_t off = row_offset<PAGED, RB>(pm, sm_pages, loc.b, g, Hkv, cap_pad, row0, r);
            kr[u] = load16_stream(Kb + off);
            vr[u] = load16_stream(Vb + off);
        }
        float s[U][GROUP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            unpack<ESZ>(kr[u], kf);
            const bool valid = full || r0 + u * RPI + sub < row_end;
#pragma unroll
            for (int i = 0; i < GROUP; ++i) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; e += 4) {
                    d = fmaf(qv[i][e / 4].x, kf[e + 0], d);
                    d = fmaf(qv[i][e / 4].y, kf[e + 1], d);
                    d = fmaf(qv[i][e / 4].z, kf[e + 2], d);
                    d = fmaf(qv[i][e / 4].w, kf[e + 3], d);
                }
                d = row_sum<LPR>(d) * qscale;
                s[u][i] = valid ? d : -INFINITY;
            }
        }
        float vf[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack<ESZ>(vr[u], vf[u]);
#pragma unroll
        for (int i = 0; i < GROUP; ++i) {
            float mx = s[0][i];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][i]);
            const float mn = fmaxf(m[i], mx);
            const float alpha = fast_exp2(m[i] - mn);
            m[i] = mn;
            float p[U];
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = fast_exp2(s[u][i] - mn);
                ps += p[u];
            }
            l[i] = fmaf(l[i], alpha, ps);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float acc = o[i][e] * alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) acc = fmaf(p[u], vf[u][e], acc);
                o[i][e] = acc;
            }
        }
    }

    // Merge the RPI row slots of the wave (lanes with equal `part`): at each
    // step a lane and its partner lane ^ msk combine the same (lower lane,
    // upper lane) pair, moved without LDS.
    auto merge_step = [&](auto pair) {
#pragma unroll
        for (int i = 0; i < GROUP; ++i) {
            float m0, m1, l0, l1;
            pair(m[i], m0, m1);
            pair(l[i], l0, l1);
            const float mn = fmaxf(m0, m1);
            const float a0 = fast_exp2(m0 - mn), a1 = fast_exp2(m1 - mn);
            l[i] = l0 * a0 + l1 * a1;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float o0, o1;
                pair(o[i][e], o0, o1);
                o[i][e] = o0 * a0 + o1 * a1;
            }
            m[i] = mn;
        }
    };
    if constexpr (LPR == 8)
        merge_step([lane](float x, float& x0, float& x1) { lane_pair8(x, lane, x0, x1); });
    merge_step([](float x, float& x0, float& x1) { lane_pair16(x, x0, x1); });
    merge_step([](float x, float& x0, float& x1) { lane_pair32(x, x0, x1); });

    // Merge the waves through LDS, then write the output (single-chunk
    // sequence) or the chunk partial.
    __shared__ float sm_o[WAVES][GROUP][kHeadDim];
    __shared__ float sm_m[WAVES][GROUP];
    __shared__ float sm_l[WAVES][GROUP];
    if (sub == 0) {
#pragma unroll
        for (int i = 0; i < GROUP; ++i) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_o[wave][i][part * EPL + e] = o[i][e];
            if (part == 0) {
                sm_m[wave][i] = m[i];
                sm_l[wave][i] = l[i];
            }
        }
    }
    finish_block<WAVES, GROUP>(sm_o, sm_m, sm_l, wave, lane, loc, g, Hq, pos.slot, out, part_o,
                               part_ml);
}

// ---------------------------------------------------------------------------
// attend, grouped-query heads on MFMA (bf16 K/V, GROUP = 2..8 query heads per
// KV head; the 16 MFMA columns / rows hold head (index mod GROUP)).
//
// Per wave iteration: 32 KV rows = two 16-row tiles.  Lane l = 16G + i.
//  loads   K and V rows as whole 128-byte rows (a wave load covers 8 full
//          rows), staged in LDS per wave: K at a 144-byte row stride, V at 160
//          (stride choices keep the 16-byte K reads and the V transpose reads
//          free of bank conflicts).  Software-pipelined: the next 32 rows are
//          requested as soon as the current ones are in LDS.  That keeps 32
//          more VGPRs live through the math, so the kernel asks the compiler
//          for 4 waves per SIMD (amdgpu_waves_per_eu), the occupancy its
//          39 KB of LDS allows anyway; it then fits in 128 registers.
//  scores  S^T = K q^T on v_mfma_f32_16x16x32_bf16: A = K tile (row i, dims
//          8G..8G+7 and 32+8G.., read back from LDS), B = the group's q
//          (column i is head i % GROUP) as bf16 hi + lo parts, so the scores
//          keep ~f32 accuracy.  Lane l receives head (l % 16) % GROUP for rows
//          4G .. 4G+3 of each tile.
//  softmax online per 32 rows; tile max per head across the four G groups.
//  P.V     O = P V on the same MFMA: A = P (row m of A is head m % GROUP, k-slot
//          8G+t <-> tile t/4, row 4G + t%4 -- exactly the lane's own eight
//          weights, in bf16 hi + lo), B = V from LDS with the gfx950 transpose
//          read ds_read_b64_tr_b16 (V rows staged row-major, 160-byte row
//          stride), four 16-dim column blocks.  The accumulator is 16 floats
//          per lane: output row 4G + r (head (4G + r) % GROUP), dim 16c + i.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int kGqaLdsStride = 160;     // bytes per staged V row (conflict-free tr16 reads)
constexpr int kGqaKStride = 144;       // bytes per staged K row (conflict-free 16-byte reads)

template <int GROUP, int WAVES, bool PAGED, int LM, bool X2>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void attend_gqa_mfma_kernel(
    const float* __restrict__ q, const char* __restrict__ K, const char* __restrict__ V,
    LensSrc<LM> ls, int B, int Hkv, int cap_pad, int row_limit, int T, int one_chunk, int uniform,
    float qscale, float* __restrict__ out, float* __restrict__ part_o, float2* __restrict__ part_ml,
    PageMap pm, CrossPart xp, Placement pl)
{
    static_assert(!(X2 && PAGED), "the one-launch layer step reads contiguous caches");
    static_assert(GROUP >= 2 && GROUP <= 8, "MFMA path takes 2..8 query heads per KV head");
    constexpr int RB = 128;                // bf16 row bytes
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int G = lane >> 4;
    const int hl = i % GROUP;              // head whose scores this lane holds
    BlockPos pos = block_pos<X2>(xp, Hkv, PAGED ? 0 : uniform);
    Located loc;
    const int is_placed = placed<LM, X2>(pl, ls, row_limit, pos, loc);
    if (is_placed < 0) return;
    const int g = pos.g;
    const int Hq = Hkv * GROUP;

    // per-wave staging of V (then K) rows; after the loop the same LDS holds
    // the per-wave partial outputs for the workgroup merge
    constexpr int kStage = 32 * (kGqaLdsStride + kGqaKStride);
    static_assert(kStage * WAVES >= static_cast<int>(sizeof(float)) * WAVES * GROUP * kHeadDim,
                  "merge area must fit in the staging LDS");
    __shared__ __attribute__((aligned(16))) char sm_stage[WAVES * kStage];

    const bool in_cross = pos.in_cross;     // workgroup-uniform
    if (in_cross) {
        const LensSrc<kLensDevice> xs{xp.lens};
        if (!locate<kLensDevice>(xs, B, xp.T, xp.row_limit, pos.blk, lane, xp.one_chunk, xp.uniform,
                                 loc))
            return;
        q = xp.q;
        K = xp.K;
        V = xp.V;
        out = xp.out;
        cap_pad = xp.cap_pad;
        T = xp.T;
    } else {
        if (!is_placed && !locate<LM>(ls, B, T, row_limit, pos.blk, lane, one_chunk, uniform, loc))
            return;
    }
    const int row0 = loc.c * T;
    int row_end = min(loc.len, row0 + T);   // lowered where a replayed row has no page

    __shared__ int sm_pages[PAGED ? kMaxChunkPages : 1];
    if constexpr (LM == kLensPagedFused)
        stage_pages<PAGED>(pm, loc.b, row0, row_end, sm_pages,
                           ls.fresh[loc.b] >= 0 ? (ls.v[loc.b] >> pm.pshift) : -1, ls.fresh[loc.b]);
    else
        stage_pages<PAGED>(pm, loc.b, row0, row_end, sm_pages);
    const char* Kb = K + 16 * (lane & 7); // + row offset, row = r0 + 8c + (lane >> 3)
    const char* Vb = V + 16 * (lane & 7);
    FreshRow<RB> fr(K, V);
    if constexpr (LM == kLensPagedFused) {
        fused_append_paged<RB>(ls, loc, g, Hkv, pm, sm_pages, row0, row_end);
    } else if constexpr (PAGED && LM == kLensDeviceFused) {
        fused_append_paged_device<RB>(ls, loc, g, Hkv, pm, sm_pages, row0, row_end);
    } else if constexpr (LM != kLensDevice) {
        if (!in_cross) fr = fresh_row<RB>(ls, loc, g, Hkv, cap_pad, row0, row_end);
    }

    // q loads, then the wave's first 32 rows, both in flight before either is
    // waited for.  The loop is software-pipelined: once a tile sits in LDS
    // its registers take the next tile's loads, which overlap the MFMA and
    // softmax work on the current one.
    // The group's q rows (GROUP x 64 floats, contiguous) come in with one
    // 16-byte load per lane per 64 float4s; the MFMA operand layout below
    // then takes each lane's 16 floats from the lanes that hold them
    // (ds_bpermute).  Loading the operand layout directly would move each
    // float4 four times per wave through the CU's in-order vector memory
    // path, whose time the K/V stream shares.
    constexpr int QN = (16 * GROUP + 63) / 64;     // float4 loads per lane
    float4 qw[QN];
    {
        const float4* qg =
            reinterpret_cast<const float4*>(q + (static_cast<size_t>(loc.b) * Hq + g * GROUP) * kHeadDim);
#pragma unroll
        for (int k = 0; k < QN; ++k) qw[k] = qg[min(64 * k + lane, 16 * GROUP - 1)];
    }
    uint4 kw[4], vr[4];
    auto load_tile = [&](int r0) {
        if (!PAGED && r0 + 32 <= row_end && (fr.row < r0 || fr.row >= r0 + 32)) {
            // whole tile inside the chunk (wave-uniform): rows r0 + 8c + lane/8
            // are 1 KB apart, no clamping
            const size_t off = row_offset<false, RB>(pm, sm_pages, loc.b, g, Hkv, cap_pad, row0,
                                                     r0 + (lane >> 3));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kw[c] = load16_stream(Kb + off + 8 * RB * c);
                vr[c] = load16_stream(Vb + off + 8 * RB * c);
            }
        } else {
            // last tile (or the one holding the new row's slot): rows past
            // the end repeat the last row (its weight is zero, and the V row
            // is finite)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = min(r0 + 8 * c + (lane >> 3), row_end - 1);
                const size_t off = row_offset<PAGED, RB>(pm, sm_pages, loc.b, g, Hkv, cap_pad, row0, r);
                kw[c] = load16_stream(fr.pick_k(r, 16 * (lane & 7), Kb + off));
                vr[c] = load16_stream(fr.pick_v(r, 16 * (lane & 7), Vb + off));
            }
        }
    };
    int r0 = row0 + wave * 32;
    if constexpr (PAGED) {
        if (r0 < row_end) load_tile(r0);
    } else {
        // The first tile is requested by every wave on one path (rows
        // clamped to the chunk's last row, or to row 0 of the stream for an
        // empty one; a wave with no rows discards what it read), so that
        // the wait for q below is a wait for the q loads alone rather than
        // for every load of the branches it joins.
        const int rmax = max(row_end - 1, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = min(r0 + 8 * c + (lane >> 3), rmax);
            const size_t off = row_offset<false, RB>(pm, sm_pages, loc.b, g, Hkv, cap_pad, row0, r);
            kw[c] = load16_stream(fr.pick_k(r, 16 * (lane & 7), Kb + off));
            vr[c] = load16_stream(fr.pick_v(r, 16 * (lane & 7), Vb + off));
        }
        // keep the scheduler from moving these loads behind the wait for q
        __builtin_amdgcn_sched_barrier(0);
        fr.store();
    }

    // B operand of the score MFMA: column i is head i % GROUP; k-slot 8G+e of
    // instruction t is dim 32t + 8G + e, i.e. float4s 16 hl + 8t + 2G and the
    // next of the group's q, held by lane (that index) % 64 of load (index) / 64.
    float4 qraw[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int F = 16 * hl + 8 * t + 2 * G + u;
            const int src = (F & 63) << 2;
            float x[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < QN; ++k) {
                    const float w = __int_as_float(__builtin_amdgcn_ds_bpermute(
                        src, __float_as_int(c == 0 ? qw[k].x : c == 1 ? qw[k].y : c == 2 ? qw[k].z : qw[k].w)));
                    v = (F >> 6) == k ? w : v;
                }
                x[c] = v;
            }
            qraw[t][u] = make_float4(x[0], x[1], x[2], x[3]);
        }
    bf16x8 qb_hi[2], qb_lo[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float4 x0 = qraw[t][0], x1 = qraw[t][1];
        const f32x8 xs = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        split_bf16(xs * qscale, qb_hi[t], qb_lo[t]);
    }

    char* my_v = sm_stage + wave * kStage;
    char* my_k = my_v + 32 * kGqaLdsStride;
    // transpose-read addresses: lane m = 4e + q of group G reads row 4G + e,
    // dims d0 + 4q .. +4 (d0 added per column block), for the second half +16 rows
    const int tr_off = (4 * G + (i >> 2)) * kGqaLdsStride + 8 * (i & 3);

    float m = kNegBig, lpart = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    while (r0 < row_end) {
        // stage K rows r0 .. r0+31, then read the A operand: row 16*tile + i,
        // bytes 16G .. and 64 + 16G ..
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint4*>(my_k + (8 * c + (lane >> 3)) * kGqaKStride + 16 * (lane & 7)) = kw[c];
        // stage V rows r0 .. r0+31 (row-major) for the transpose reads
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint4*>(my_v + (8 * c + (lane >> 3)) * kGqaLdsStride + 16 * (lane & 7)) = vr[c];
        uint4 kr[2][2];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const char* kp = my_k + (16 * tile + i) * kGqaKStride + 16 * G;
            kr[tile][0] = *reinterpret_cast<const uint4*>(kp);
            kr[tile][1] = *reinterpret_cast<const uint4*>(kp + 64);
        }
        const int rn = r0 + WAVES * 32;
        if (rn < row_end) load_tile(rn);
        // scores: lane holds head hl for rows r0 + 16*tile + 4G + rr
        float sc[2][4];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, kr[tile][t]);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb_hi[t], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb_lo[t], c, 0, 0, 0);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sc[tile][rr] = c[rr];
        }
        if (r0 + 32 > row_end) {           // last tile of the chunk (wave-uniform)
#pragma unroll
            for (int tile = 0; tile < 2; ++tile)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    if (r0 + 16 * tile + 4 * G + rr >= row_end) sc[tile][rr] = -INFINITY;
        }

        // online softmax for head hl over these 32 rows
        const float mx = max_over_groups(
            fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                  fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3]))));
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        float pw[2][4];
        float ps = 0.f;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                pw[tile][rr] = fast_exp2(sc[tile][rr] - mn);
                ps += pw[tile][rr];
            }
        lpart = fmaf(lpart, alpha, ps);
        // A operand of P.V: k-slot 8G + t <-> tile t / 4, row 4G + t % 4
        bf16x8 pa_hi, pa_lo;
        split_bf16(f32x8{pw[0][0], pw[0][1], pw[0][2], pw[0][3], pw[1][0], pw[1][1], pw[1][2], pw[1][3]},
                   pa_hi, pa_lo);
        // rescale the accumulator: output row 4G + rr is head (4G + rr) % GROUP,
        // whose alpha lane (4G + rr) % GROUP holds (its column is that head)
        float ah[GROUP];                   // alpha of every head, wave-uniform
#pragma unroll
        for (int h = 0; h < GROUP; ++h)
            ah[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
        float al[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            al[rr] = G == 0 ? ah[rr % GROUP]
                   : G == 1 ? ah[(4 + rr) % GROUP]
                   : G == 2 ? ah[(8 + rr) % GROUP] : ah[(12 + rr) % GROUP];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) o[c][rr] *= al[rr];
        // P.V, one 16-dim column block at a time
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
            typedef __attribute__((address_space(3))) char lds_char;
            lds_char* base = (lds_char*)(my_v) + tr_off + 32 * c;
            const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base));
            const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(base + 16 * kGqaLdsStride));
            const v8i16 vv = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 vb = __builtin_bit_cast(bf16x8, vv);
            o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb, o[c], 0, 0, 0);
            o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb, o[c], 0, 0, 0);
        }
        r0 = rn;
    }

    // l: sum over the four G groups (lanes whose columns repeat a head repeat it)
    lpart = sum_over_groups(lpart);

    // every wave must be done with its staging LDS before it becomes sm_o
    __syncthreads();
    auto& sm_o = *reinterpret_cast<float (*)[WAVES][GROUP][kHeadDim]>(sm_stage);
    __shared__ float sm_m[WAVES][GROUP];
    __shared__ float sm_l[WAVES][GROUP];
    // output rows 0 .. GROUP-1 are the heads; later rows repeat them
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        if (4 * G + rr < GROUP) {
#pragma unroll
            for (int c = 0; c < 4; ++c) sm_o[wave][4 * G + rr][16 * c + i] = o[c][rr];
        }
    }
    if (lane < GROUP) {
        sm_m[wave][lane] = m;
        sm_l[wave][lane] = lpart;
    }
    finish_block<WAVES, GROUP>(sm_o, sm_m, sm_l, wave, lane, loc, g, Hq, pos.slot, out, part_o,
                               part_ml);
}

// ---------------------------------------------------------------------------
// merge: one wave per (sequence, query head).  Lane c takes chunk c's (m, l)
// to form the global max M and the weights w_c = 2^(m_c - M); lane d sums
// w_c * o_c[d] over the chunks in chunk order (a fixed order: the result does
// not depend on scheduling).  The kernel is latency-bound (a few KB per
// wave), so the loads are grouped to keep the chain of dependent round trips
// short: lengths -> {(m, l), first 16 o rows} -> further batches of 16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_core(size_t first, int nch, int Hq, int h, int lane,
                                           const float* __restrict__ part_o,
                                           const float2* __restrict__ part_ml,
                                           float* __restrict__ out_row);

// One (sequence b, query head h) of one part of the grid: its chunks'
// partials start at slot `base` + the exclusive prefix of the part's chunk
// counts; n_grid is the number of workgroups the part was launched with.
template <int LM>
__device__ __forceinline__ void merge_one(const LensSrc<LM>& ls, int B, int Hq, int T,
                                          int row_limit, int b, int h, int lane, int base,
                                          int n_grid, const float* __restrict__ part_o,
                                          const float2* __restrict__ part_ml,
                                          float* __restrict__ out, const PageMap& pm)
{
    constexpr int plus = LensSrc<LM>::kPlus;
    const size_t w = static_cast<size_t>(b) * Hq + h;
    // exclusive prefix of chunk counts over sequences < b, and this sequence's count
    int acc = 0;
    for (int b0 = 0; b0 < b; b0 += 64) {
        const int bi = b0 + lane;
        if (bi < b) acc += max(1, (min(max(ls.merge_get(bi) + plus, 0), row_limit) + T - 1) / T);
    }
    acc = wave_sum_int(acc);
    const int len0 = ls.merge_get(b);
    const int nch = max(1, (min(max(len0 + plus, 0), row_limit) + T - 1) / T);
    // a replay grid sized with a horizon that the lengths have outgrown ends
    // before this sequence's last chunk: no length bump, NaN rows
    const bool covered = acc + nch <= n_grid;
    if constexpr (LM == kLensDeviceFused) {
        // the device-fused append's length bump (refused, like kvdec_append,
        // when a linear cache is full: row_limit is its capacity)
        // (and, in a paged cache, when the new row had no page)
        if (covered && h == 0 && lane == 0 && (ls.f.window > 0 || len0 < row_limit) &&
            (!pm.table || pm.table[static_cast<size_t>(b) * pm.stride + (len0 >> pm.pshift)] >= 0))
            ls.f.lens_out[b] = len0 + 1;
    }
    if (!covered) {
        out[w * kHeadDim + lane] = __int_as_float(0x7fc00000);
        return;
    }
    if (nch == 1) return;     // finished by the attend kernel
    merge_core(static_cast<size_t>(base) + static_cast<size_t>(acc), nch, Hq, h, lane, part_o,
               part_ml, out + w * kHeadDim);
}

// The merge of one (sequence, query head) whose nch chunk partials start at
// slot `first`, into the output row out_row[64].
__device__ __forceinline__ void merge_core(size_t first, int nch, int Hq, int h, int lane,
                                           const float* __restrict__ part_o,
                                           const float2* __restrict__ part_ml,
                                           float* __restrict__ out_row)
{
    // Chunk c's (m, l) is read by lane c % 64; the o rows are read kBatch
    // chunks at a time, all loads of a batch in flight together, and the
    // first batch is issued with the (m, l) loads (it does not need M).
    // Indices past the last chunk are clamped (their values are not used).
    constexpr int kBatch = 16;
    float ov[kBatch];
    auto load_batch = [&](int cb) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const size_t c = first + min(cb + j, nch - 1);
            ov[j] = part_o[(c * Hq + h) * kHeadDim + lane];
        }
    };
    float2 ml0 = make_float2(kNegBig, 0.f);
    if (lane < nch) ml0 = part_ml[(first + lane) * Hq + h];
    load_batch(0);

    // global max over the chunks' m (lane-parallel)
    float M = ml0.x;
    for (int c0 = 64; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        if (c < nch) M = fmaxf(M, part_ml[(first + c) * Hq + h].x);
    }
    M = max_over_groups(row_max16(M));

    // weights w_c = 2^(m_c - M); sums of w_c l_c and w_c o_c in chunk order
    float Lsum = 0.f, o = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        float2 ml = ml0;
        if (c0 > 0) ml = c < nch ? part_ml[(first + c) * Hq + h] : make_float2(kNegBig, 0.f);
        const float wc = c < nch ? fast_exp2(ml.x - M) : 0.f;
        const float lc = c < nch ? ml.y : 0.f;
        const int n = min(64, nch - c0);
        for (int k0 = 0; k0 < n; k0 += kBatch) {
            if (c0 + k0 > 0) load_batch(c0 + k0);
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (k0 + j < n) {
                    // chunk c0 + k0 + j's weight and l, from its lane (scalar reads)
                    const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wc), k0 + j));
                    const float lk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lc), k0 + j));
                    Lsum = fmaf(lk, wk, Lsum);
                    o = fmaf(ov[j], wk, o);
                }
            }
        }
    }
    out_row[lane] = (Lsum > 0.f) ? o / Lsum : 0.f;
}

// One wave per (sequence, query head) of the launch's part(s): waves
// [0, B*Hq) merge the self part (whose partials follow the cross part's in
// a one-launch layer step), waves [B*Hq, 2*B*Hq) the cross part.
template <int LM, bool X2>
__global__ __launch_bounds__(64) void merge_kernel(LensSrc<LM> ls, int B, int Hq,
                                                    int T, int row_limit,
                                                    const float* __restrict__ part_o,
                                                    const float2* __restrict__ part_ml,
                                                    float* __restrict__ out, PageMap pm,
                                                    int n_grid, CrossPart xp)
{
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x;
    if (X2 && w >= B * Hq) {
        const int wx = w - B * Hq;
        if (wx >= B * Hq) return;
        const int b = wx / Hq, h = wx - b * Hq;
        const LensSrc<kLensDevice> xs{xp.lens};
        merge_one<kLensDevice>(xs, B, Hq, xp.T, xp.row_limit, b, h, lane, 0, xp.n_blocks, part_o,
                               part_ml, xp.out, PageMap{nullptr, 0, 0, 0});
        return;
    }
    if (w >= B * Hq) return;
    const int b = w / Hq, h = w - b * Hq;
    merge_one<LM>(ls, B, Hq, T, row_limit, b, h, lane, X2 ? xp.n_blocks : 0, n_grid, part_o, part_ml,
                  out, pm);
}

// The merge where the host knows every sequence's chunk count (outside
// replay mode the grids are sized from lengths the host holds): one wave per
// (split sequence, query head), the sequence's first partial slot and chunk
// count given by value, so no wave reads a length or scans the other
// sequences' chunk counts, and no wave is launched for a sequence that the
// attend launch finished in place.
__global__ __launch_bounds__(64) void merge_planned_kernel(MergePlan plan, int Hq,
                                                           const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           float* __restrict__ out,
                                                           float* __restrict__ out_x)
{
    const int lane = threadIdx.x & 63;
    const int e = static_cast<int>(blockIdx.x) / Hq;
    const int h = static_cast<int>(blockIdx.x) - e * Hq;
    const int nch = plan.nch[e] & 0xFFFFFF;
    float* o = (plan.nch[e] >> 24) ? out_x : out;
    merge_core(static_cast<size_t>(plan.first[e]), nch, Hq, h, lane, part_o, part_ml,
               o + (static_cast<size_t>(plan.b[e]) * Hq + h) * kHeadDim);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
PartialLayout partial_layout(int64_t max_chunks, int32_t n_q_heads, int32_t batch)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    PartialLayout p;
    const size_t slots = static_cast<size_t>(max_chunks) * static_cast<size_t>(n_q_heads);
    p.o_offset = 0;
    p.ml_offset = up(slots * kHeadDim * sizeof(float));
    p.snap_offset = p.ml_offset + up(slots * sizeof(float2));
    p.bytes = p.snap_offset + up(static_cast<size_t>(batch) * sizeof(int32_t));
    return p;
}

hipError_t launch_set_lens(int32_t* lens, const int32_t* host, int32_t n, hipStream_t s)
{
    for (int32_t off = 0; off < n; off += kLensPerLaunch) {
        LensBlock blk;
        const int32_t cnt = (n - off) < kLensPerLaunch ? (n - off) : kLensPerLaunch;
        for (int32_t i = 0; i < kLensPerLaunch; ++i) blk.v[i] = i < cnt ? host[off + i] : 0;
        hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(kLensPerLaunch), 0, s, lens + off, cnt,
                           blk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_append(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                         int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                         int32_t cap_pad, int32_t window, hipStream_t s)
{
    const dim3 grid(batch), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(append_kernel<256>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad, window);
    else
        hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad, window);
    return hipGetLastError();
}

hipError_t launch_append_slide(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                               int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                               int32_t cap_pad, int32_t keep, hipStream_t s)
{
    const dim3 grid(batch), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(append_slide_kernel<256>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad, keep);
    else
        hipLaunchKernelGGL(append_slide_kernel<128>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad, keep);
    return hipGetLastError();
}

hipError_t launch_append_rope(int dtype, void* k, void* v, const void* k_new, const void* v_new,
                              int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t capacity,
                              int32_t cap_pad, int32_t window, const float* q, float* q_rot,
                              int32_t n_q_heads, double theta, hipStream_t s)
{
    const dim3 grid(batch), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(append_rope_kernel<4>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad,
                           window, q, q_rot, n_q_heads, theta);
    else
        hipLaunchKernelGGL(append_rope_kernel<2>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_new),
                           static_cast<const char*>(v_new), lens, n_kv_heads, capacity, cap_pad,
                           window, q, q_rot, n_q_heads, theta);
    return hipGetLastError();
}

hipError_t launch_paged_append(int dtype, void* k_pages, void* v_pages, const void* k_new,
                               const void* v_new, int32_t* lens, int32_t* table,
                               int32_t table_stride, int32_t batch, int32_t n_kv_heads,
                               int32_t pshift, int32_t num_pages, const int32_t* new_pages,
                               bool from_table, hipStream_t s)
{
    for (int32_t b0 = 0; b0 < batch; b0 += kPagesPerLaunch) {
        const int32_t cnt = (batch - b0) < kPagesPerLaunch ? (batch - b0) : kPagesPerLaunch;
        PageBlock blk;
        for (int32_t i = 0; i < kPagesPerLaunch; ++i) blk.v[i] = i < cnt ? new_pages[b0 + i] : -1;
        const dim3 grid(cnt), block(256);
        if (dtype == 0)
            hipLaunchKernelGGL(paged_append_kernel<256>, grid, block, 0, s,
                               static_cast<char*>(k_pages), static_cast<char*>(v_pages),
                               static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                               lens, table, table_stride, n_kv_heads, pshift, num_pages, b0, blk,
                               from_table ? 1 : 0);
        else
            hipLaunchKernelGGL(paged_append_kernel<128>, grid, block, 0, s,
                               static_cast<char*>(k_pages), static_cast<char*>(v_pages),
                               static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                               lens, table, table_stride, n_kv_heads, pshift, num_pages, b0, blk,
                               from_table ? 1 : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_paged_reserve(int32_t* table, int32_t table_stride, int32_t* lens, int32_t seq,
                                const int32_t* pages, int32_t n_pages, int32_t len, hipStream_t s)
{
    const size_t base = static_cast<size_t>(seq) * table_stride;
    for (int32_t off = 0; off < n_pages || (off == 0 && n_pages == 0); off += kPagesPerLaunch) {
        const int32_t cnt = (n_pages - off) < kPagesPerLaunch ? (n_pages - off) : kPagesPerLaunch;
        PageBlock blk;
        for (int32_t i = 0; i < kPagesPerLaunch; ++i) blk.v[i] = i < cnt ? pages[off + i] : -1;
        // the length is written by the last launch, after every table entry
        const bool last = off + kPagesPerLaunch >= n_pages;
        hipLaunchKernelGGL(paged_reserve_kernel, dim3(1), dim3(kPagesPerLaunch), 0, s, table + base,
                           lens, seq, off, cnt, last ? len : -1, blk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (n_pages == 0) break;
    }
    return hipSuccess;
}

hipError_t launch_table_clear_tail(int32_t* table, int32_t table_stride, const int32_t* held,
                                   int32_t batch, hipStream_t s)
{
    for (int32_t b0 = 0; b0 < batch; b0 += kLensPerLaunch) {
        const int32_t cnt = (batch - b0) < kLensPerLaunch ? (batch - b0) : kLensPerLaunch;
        LensBlock blk;
        for (int32_t i = 0; i < kLensPerLaunch; ++i) blk.v[i] = i < cnt ? held[b0 + i] : table_stride;
        hipLaunchKernelGGL(table_clear_tail_kernel, dim3(cnt), dim3(64), 0, s, table, table_stride, b0,
                           blk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)),
                       dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_table_write(int32_t* table, const int32_t* idx, const int32_t* val, int32_t n,
                              hipStream_t s)
{
    for (int32_t off = 0; off < n; off += kEntriesPerLaunch) {
        const int32_t cnt = (n - off) < kEntriesPerLaunch ? (n - off) : kEntriesPerLaunch;
        EntryBlock blk;
        for (int32_t i = 0; i < kEntriesPerLaunch; ++i) {
            blk.idx[i] = i < cnt ? idx[off + i] : 0;
            blk.val[i] = i < cnt ? val[off + i] : 0;
        }
        hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(kEntriesPerLaunch), 0, s, table, cnt, blk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_seed(int dtype, void* k, void* v, const void* k_tok, const void* v_tok,
                       int32_t batch, int32_t rows, int32_t n_kv_heads, int32_t cap_pad,
                       hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    const size_t words = static_cast<size_t>(batch) * rows * n_kv_heads * (dtype == 0 ? 16 : 8) * 2;
    size_t blocks = (words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(seed_kernel<256>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_tok),
                           static_cast<const char*>(v_tok), batch, rows, n_kv_heads, cap_pad);
    else
        hipLaunchKernelGGL(seed_kernel<128>, grid, block, 0, s, static_cast<char*>(k),
                           static_cast<char*>(v), static_cast<const char*>(k_tok),
                           static_cast<const char*>(v_tok), batch, rows, n_kv_heads, cap_pad);
    return hipGetLastError();
}

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

constexpr int kWideWaves = 16;

// Whether two 16-wave workgroups of the f32 VALU kernel for GROUP fit on a
// CU (occupancy query of the plain contiguous instance, once).  The answer
// depends on the kernel alone, never on the launch, so every call with the
// same chunk size picks the same wave count: a sequence's rows are split
// over waves and row slots the same way whatever else is in the batch, and
// in the fused and unfused forms alike (the two wave counts sum a chunk's
// rows in different orders, so they differ in the last bits).
template <int GROUP>
bool wide_fits()
{
    static std::atomic<int> known{0};       // 0: not asked yet, 1: fits, -1: does not
    int k = known.load(std::memory_order_relaxed);
    if (k == 0) {
        int per_cu = 0;
        const bool ok =
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu,
                reinterpret_cast<const void*>(&attend_kernel<4, GROUP, kWideWaves, kUnroll, false,
                                                             kLensDevice, false>),
                kWideWaves * 64, 0) == hipSuccess;
        k = (ok && per_cu >= 2) ? 1 : -1;
        known.store(k, std::memory_order_relaxed);
    }
    return k > 0;
}

// f32 with 1 or 2 query heads per KV head: chunks of >= 256 rows run on
// 16-wave workgroups (each wave one pass of 16 rows per 256 rows) where two
// of them fit on a CU.  The choice depends on the chunk size and the kernel
// only (see wide_fits), not on the grid.  Not for capacity-sized replay
// grids: there a surplus workgroup launches and retires 16 waves for nothing
// (qwen2-0.5b replayed: 83.3 us per step on 16-wave, 80.1 on 4-wave
// workgroups).
template <int ESZ, int GROUP>
bool use_wide(int chunk_rows, bool replay)
{
    if constexpr (ESZ == 4 && GROUP <= 2)
        return !replay && chunk_rows >= kWideWaves * kUnroll * Lay<4>::kRPI && wide_fits<GROUP>();
    else
        return false;
}

CrossPart cross_part(const AttendArgs& a)
{
    CrossPart x{};
    if (a.x_blocks > 0) {
        x.q = a.x_q;
        x.K = static_cast<const char*>(a.x_k);
        x.V = static_cast<const char*>(a.x_v);
        x.lens = a.x_lens;
        x.out = a.x_out;
        x.cap_pad = a.x_cap_pad;
        x.row_limit = a.x_row_limit;
        x.T = a.x_chunk_rows;
        x.one_chunk = a.x_one_chunk;
        x.uniform = a.x_uniform;
        x.n_blocks = static_cast<int>(a.x_blocks);
    }
    return x;
}

// The merge launch after an attend launch, when some sequence of some part
// spans several chunks.
template <int LM, bool X2>
hipError_t launch_merge(const AttendArgs& a, int group, const LensSrc<LM>& ls, float* po,
                        float2* pml, const PageMap& pm, const CrossPart& xp, hipStream_t s)
{
    if (!a.need_merge) return hipSuccess;
    const int Hq = a.n_kv_heads * group;
    if (a.merge_plan) {
        // the host planned it: only the split sequences, their slots by value
        if (a.merge_plan->n == 0) return hipSuccess;
        hipLaunchKernelGGL(merge_planned_kernel, dim3(a.merge_plan->n * Hq), dim3(64), 0, s,
                           a.merge_plan->plan, Hq, po, pml, a.out, a.x_out);
        return hipGetLastError();
    }
    const int waves = a.batch * Hq * (X2 ? 2 : 1);
    // one wave per workgroup: the waves spread over more CUs (whisper-base
    // 27.3 -> 26.6 us per step against four-wave workgroups)
    hipLaunchKernelGGL((merge_kernel<LM, X2>), dim3(waves), dim3(64), 0, s, ls, a.batch,
                       Hq, a.chunk_rows, a.row_limit, po, pml, a.out, pm,
                       static_cast<int>(a.n_chunks), xp);
    return hipGetLastError();
}

template <int ESZ, int GROUP, bool PAGED, int LM, bool X2>
hipError_t attend_t(const AttendArgs& a, hipStream_t s)
{
    char* ws = static_cast<char*>(a.ws);
    float* po = reinterpret_cast<float*>(ws + a.part.o_offset);
    float2* pml = reinterpret_cast<float2*>(ws + a.part.ml_offset);
    const PageMap pm{a.table, a.table_stride, a.pshift, a.num_pages};
    const CrossPart xp = cross_part(a);
    LensSrc<LM> ls;
    if constexpr (LM == kLensDevice) {
        ls.lens = a.lens;
    } else if constexpr (LM == kLensPagedFused) {
        for (int b = 0; b < kMaxPagedFusedBatch; ++b) {
            ls.v[b] = b < a.batch ? a.fused_lens[b] : 0;
            ls.fresh[b] = b < a.batch ? a.fresh_pages[b] : -1;
        }
        ls.f.k_new = static_cast<const char*>(a.k_new);
        ls.f.v_new = static_cast<const char*>(a.v_new);
        ls.f.K = static_cast<char*>(const_cast<void*>(a.k));
        ls.f.V = static_cast<char*>(const_cast<void*>(a.v));
        ls.f.lens_out = a.lens_out;
        ls.f.table_out = const_cast<int32_t*>(a.table);
    } else {
        if constexpr (LM == kLensHostFused) {
            for (int b = 0; b < kMaxFusedBatch; ++b) ls.v[b] = b < a.batch ? a.fused_lens[b] : 0;
        } else {
            ls.lens = a.lens;
            ls.snap = reinterpret_cast<int32_t*>(ws + a.part.snap_offset);
        }
        ls.f.k_new = static_cast<const char*>(a.k_new);
        ls.f.v_new = static_cast<const char*>(a.v_new);
        ls.f.K = static_cast<char*>(const_cast<void*>(a.k));
        ls.f.V = static_cast<char*>(const_cast<void*>(a.v));
        ls.f.lens_out = a.lens_out;
        ls.f.window = a.window;
    }
    // with a cross part: one dimension, every cross workgroup first (see block_pos)
    // a placement (host-fused launches of the MFMA kernel): (KV head, position) grid
    Placement pl;
    pl.n = 0;
    if constexpr ((LM == kLensHostFused || LM == kLensPagedFused) && !X2 && ESZ == 2 &&
                  GROUP >= 2) {
        if (a.placement && a.placement->n > 0) {
            pl.n = a.placement->n;
            for (int i = 0; i < pl.n; ++i) pl.pos[i] = a.placement->pos[i];
        }
    }
    const dim3 grid = X2 ? dim3(static_cast<unsigned>((a.n_chunks + a.x_blocks) * a.n_kv_heads))
                    : pl.n > 0 ? dim3(a.n_kv_heads, static_cast<unsigned>(pl.n))
                    : !PAGED && a.uniform < 0 && a.n_chunks <= 65535
                          ? dim3(a.n_kv_heads, static_cast<unsigned>(a.n_chunks))
                          : dim3(static_cast<unsigned>(a.n_chunks), a.n_kv_heads);
    const dim3 block(kWaves * 64);
    if (use_wide<ESZ, GROUP>(a.chunk_rows, a.replay)) {
        if constexpr (ESZ == 4 && GROUP <= 2)
            hipLaunchKernelGGL((attend_kernel<ESZ, GROUP, kWideWaves, kUnroll, PAGED, LM, X2>), grid,
                               dim3(kWideWaves * 64), 0, s, a.q, static_cast<const char*>(a.k),
                               static_cast<const char*>(a.v), ls, a.batch, a.n_kv_heads, a.cap_pad,
                               a.row_limit, a.chunk_rows, a.one_chunk, a.uniform, a.qscale, a.out,
                               po, pml, pm, xp);
    } else if constexpr (ESZ == 2 && GROUP >= 2) {
        hipLaunchKernelGGL((attend_gqa_mfma_kernel<GROUP, kWaves, PAGED, LM, X2>), grid, block, 0, s,
                           a.q, static_cast<const char*>(a.k), static_cast<const char*>(a.v), ls,
                           a.batch, a.n_kv_heads, a.cap_pad, a.row_limit, a.chunk_rows, a.one_chunk,
                           a.uniform, a.qscale, a.out, po, pml, pm, xp, pl);
    } else {
        hipLaunchKernelGGL((attend_kernel<ESZ, GROUP, kWaves, kUnroll, PAGED, LM, X2>), grid, block,
                           0, s, a.q, static_cast<const char*>(a.k), static_cast<const char*>(a.v),
                           ls, a.batch, a.n_kv_heads, a.cap_pad, a.row_limit, a.chunk_rows,
                           a.one_chunk, a.uniform, a.qscale, a.out, po, pml, pm, xp);
    }
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_merge<LM, X2>(a, GROUP, ls, po, pml, pm, xp, s);
}

template <int ESZ, int GROUP, bool PAGED, int LM>
hipError_t attend_x(const AttendArgs& a, hipStream_t s)
{
    if constexpr (!PAGED && (LM == kLensHostFused || LM == kLensDeviceFused)) {
        if (a.x_blocks > 0) return attend_t<ESZ, GROUP, PAGED, LM, true>(a, s);
    }
    if (a.x_blocks > 0) return hipErrorInvalidValue;    // no cross part in this mode
    return attend_t<ESZ, GROUP, PAGED, LM, false>(a, s);
}

template <int ESZ, bool PAGED, int LM>
hipError_t attend_dispatch_group(const AttendArgs& a, hipStream_t s)
{
    switch (a.group) {
        case 1: return attend_x<ESZ, 1, PAGED, LM>(a, s);
        case 2: return attend_x<ESZ, 2, PAGED, LM>(a, s);
        case 3: return attend_x<ESZ, 3, PAGED, LM>(a, s);
        case 4: return attend_x<ESZ, 4, PAGED, LM>(a, s);
        case 5: return attend_x<ESZ, 5, PAGED, LM>(a, s);
        case 6: return attend_x<ESZ, 6, PAGED, LM>(a, s);
        case 7: return attend_x<ESZ, 7, PAGED, LM>(a, s);
        case 8: return attend_x<ESZ, 8, PAGED, LM>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int ESZ>
int waves_for(int group, int chunk_rows, bool replay)
{
    switch (group) {
        case 1: return use_wide<ESZ, 1>(chunk_rows, replay) ? kWideWaves : kWaves;
        case 2: return use_wide<ESZ, 2>(chunk_rows, replay) ? kWideWaves : kWaves;
        default: return kWaves;
    }
}

}  // namespace

int attend_waves(int dtype, int group, int chunk_rows, bool replay)
{
    return dtype == 0 ? waves_for<4>(group, chunk_rows, replay) : waves_for<2>(group, chunk_rows, replay);
}

namespace {

template <int ESZ>
const void* attend_kernel_ptr(int group, int* block)
{
    *block = kWaves * 64;
    if constexpr (ESZ == 2) {
        switch (group) {
            case 1: return reinterpret_cast<const void*>(&attend_kernel<2, 1, kWaves, kUnroll, false, kLensDevice, false>);
            case 2: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<2, kWaves, false, kLensDevice, false>);
            case 3: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<3, kWaves, false, kLensDevice, false>);
            case 4: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<4, kWaves, false, kLensDevice, false>);
            case 5: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<5, kWaves, false, kLensDevice, false>);
            case 6: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<6, kWaves, false, kLensDevice, false>);
            case 7: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<7, kWaves, false, kLensDevice, false>);
            case 8: return reinterpret_cast<const void*>(&attend_gqa_mfma_kernel<8, kWaves, false, kLensDevice, false>);
            default: return nullptr;
        }
    } else {
        switch (group) {
            case 1: return reinterpret_cast<const void*>(&attend_kernel<4, 1, kWaves, kUnroll, false, kLensDevice, false>);
            case 2: return reinterpret_cast<const void*>(&attend_kernel<4, 2, kWaves, kUnroll, false, kLensDevice, false>);
            case 3: return reinterpret_cast<const void*>(&attend_kernel<4, 3, kWaves, kUnroll, false, kLensDevice, false>);
            case 4: return reinterpret_cast<const void*>(&attend_kernel<4, 4, kWaves, kUnroll, false, kLensDevice, false>);
            case 5: return reinterpret_cast<const void*>(&attend_kernel<4, 5, kWaves, kUnroll, false, kLensDevice, false>);
            case 6: return reinterpret_cast<const void*>(&attend_kernel<4, 6, kWaves, kUnroll, false, kLensDevice, false>);
            case 7: return reinterpret_cast<const void*>(&attend_kernel<4, 7, kWaves, kUnroll, false, kLensDevice, false>);
            case 8: return reinterpret_cast<const void*>(&attend_kernel<4, 8, kWaves, kUnroll, false, kLensDevice, false>);
            default: return nullptr;
        }
    }
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_resident[kMaxDevices][2][KVDEC_MAX_GROUP + 1];

}  // namespace

int device_cus()
{
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (n > 0) cached[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

int resident_attend_blocks(int dtype, int group)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    if (group < 1 || group > KVDEC_MAX_GROUP) return 0;
    std::atomic<int>& slot = g_resident[dev][dtype == 0 ? 0 : 1][group];
    int cached = slot.load(std::memory_order_relaxed);
    if (cached > 0) return cached;
    int block = 0;
    const void* fn = dtype == 0 ? attend_kernel_ptr<4>(group, &block) : attend_kernel_ptr<2>(group, &block);
    int per_cu = 0, cus = 0;
    if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int n = per_cu * cus;
    if (n > 0) slot.store(n, std::memory_order_relaxed);
    return n;
}

// ---------------------------------------------------------------------------
// The library's own device scratch, for the entry point that allocates
// nothing (kvdec_append_attend_noalloc): the split-sequence partials and the
// length snapshot that the caller's workspace holds otherwise.  Each GPU the
// library runs on holds one copy, at its own address, until the process
// ends; every call on that GPU shares it (the partials need no initial
// contents: each launch writes the slots it reads).  In host code `scratch`
// names a host-side stand-in, never the device memory: the address comes
// from hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[KVDEC_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_device_ptr(void** ptr, size_t* bytes)
{
    *ptr = nullptr;
    *bytes = KVDEC_NOALLOC_SCRATCH_BYTES;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_attend(int dtype, const AttendArgs& a, hipStream_t s)
{
    if (a.table && a.fresh_pages) {
        if (a.batch > kMaxPagedFusedBatch || !a.fused_lens) return hipErrorInvalidValue;
        return dtype == 0 ? attend_dispatch_group<4, true, kLensPagedFused>(a, s)
                          : attend_dispatch_group<2, true, kLensPagedFused>(a, s);
    }
    if (a.table && a.fused_device) {
        if (!a.need_merge) return hipErrorInvalidValue;   // the merge launch bumps the lengths
        return dtype == 0 ? attend_dispatch_group<4, true, kLensDeviceFused>(a, s)
                          : attend_dispatch_group<2, true, kLensDeviceFused>(a, s);
    }
    if (a.table)
        return dtype == 0 ? attend_dispatch_group<4, true, kLensDevice>(a, s)
                          : attend_dispatch_group<2, true, kLensDevice>(a, s);
    if (a.fused_lens) {
        if (a.batch > kMaxFusedBatch) return hipErrorInvalidValue;
        return dtype == 0 ? attend_dispatch_group<4, false, kLensHostFused>(a, s)
                          : attend_dispatch_group<2, false, kLensHostFused>(a, s);
    }
    if (a.fused_device) {
        if (!a.need_merge) return hipErrorInvalidValue;   // the merge launch bumps the lengths
        return dtype == 0 ? attend_dispatch_group<4, false, kLensDeviceFused>(a, s)
                          : attend_dispatch_group<2, false, kLensDeviceFused>(a, s);
    }
    return dtype == 0 ? attend_dispatch_group<4, false, kLensDevice>(a, s)
                      : attend_dispatch_group<2, false, kLensDevice>(a, s);
}

}  // namespace kvdec
