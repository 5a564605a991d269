// Pieces shared by the two prefill kernels (prefill.hip: 32x32x2 MFMA,
// 4 waves of 32 query rows; prefill16.hip: 16x16x4 MFMA, 8 waves of 16 query
// rows): workgroup numbering, the visible key range, tile visibility, and
// the global -> LDS staging of K/V tiles.
#pragma once

#include "device_common.h"

namespace attn {
namespace pf {

constexpr int kBK = 32;       // key rows per LDS tile
constexpr int kPad = 4;       // floats of padding per LDS row (bank spread)
constexpr float kLazy = 8.0f; // log2 of the largest weight before the reference max moves
constexpr int kXcds = 8;      // MI355X: 8 XCDs of 32 CUs, each with its own L2

// Workgroup layout chosen on the host: nh heads of one KV group side by side,
// each with the rest of the workgroup's waves on consecutive query blocks, and
// ksplit key-range parts per workgroup.
struct Args {
    int nh;            // heads per workgroup
    int hgroups;       // head groups per KV head = (heads/kvHeads) / nh
    int qblocks;       // workgroups along the query rows
    int ksplit;        // parts of this launch's key tiles per workgroup
    int causal_order;  // 1: heaviest query blocks first
    float* ws;         // partial states when kslots > 1
    int part;          // key tiles of a workgroup this launch takes: 0 all; with relative
                       // embeddings 1 those beyond their reach for every row, 2 the rest
    int kslot0;        // partial-state slot of this launch's part 0
    int kslots;        // partial-state slots per row over all launches (1: write out directly)
};


struct Coords {
    int ks;   // key-range part
    int g;    // KV head
    int hgi;  // head group within the KV head
    int qb;   // query block
};

// Workgroups are dealt round-robin to the XCDs. Renumber them so that each
// XCD gets a contiguous run of (KV head, query block, key part) work: the K/V
// of a KV head then stays in one L2. Within a run the heaviest (latest, for
// causal) query blocks start first.
__device__ __forceinline__ Coords wg_coords(const Args& a) {
    const int nwg = (int)gridDim.x;
    int wid = (int)blockIdx.x;
    if (nwg % kXcds == 0) wid = (wid % kXcds) * (nwg / kXcds) + wid / kXcds;
    Coords c;
    c.ks = wid % a.ksplit;
    const int yq = wid / a.ksplit / a.qblocks;
    const int xq = wid / a.ksplit % a.qblocks;
    c.qb = a.causal_order ? (a.qblocks - 1 - xq) : xq;
    c.g = yq / a.hgroups;
    c.hgi = yq % a.hgroups;
    return c;
}

// Keys that any query row at positions [pf, pl] can see (graph protocol op
// catalogue, op `attention`, params causal and window).
__device__ __forceinline__ void visible_keys(const Epilogue& e, int S, int pf, int pl, int& klo,
                                             int& khi) {
    klo = 0;
    khi = S;
    if (e.causal) {
        khi = min(S, pl + 1);
        if (e.window > 0) klo = max(0, pf - e.window + 1);
    } else if (e.window > 0) {
        klo = max(0, pf - e.window);
        khi = (int)min((int64_t)S, (int64_t)pl + e.window + 1);
    }
}

// The key rows a workgroup loads: the attention sinks below its window range,
// [0, sink_hi), and the window range [klo, khi). Other rows are never read;
// their LDS rows are zero. 1 <= khi <= S, so clamping a row number into
// [klo, khi - 1] gives an in-bounds row whether or not the window is empty.
// Every loaded row lies below khi, and every row below khi that is not loaded
// is hidden from all the workgroup's queries (before every window, not a
// sink), so inside a tile `s < khi` and the visibility rule mask exactly.
struct KeyRows {
    int sink_hi, klo, khi;
    __device__ __forceinline__ bool loaded(int s) const {
        return ((unsigned)s < (unsigned)sink_hi) | ((unsigned)(s - klo) < (unsigned)(khi - klo));
    }
};

__device__ __forceinline__ KeyRows key_rows(const Epilogue& e, int klo, int khi) {
    KeyRows r;
    r.sink_hi = min(e.sinks, klo);  // e.sinks is 0 without a window
    r.klo = klo;
    r.khi = khi;
    return r;
}

// The workgroup's key tiles in the order it visits them: the sink tiles
// [0, nst), then the window tiles from kt_w0. Virtual tile v is tile
// v < nst ? v : kt_w0 + v - nst.
struct TileSpan {
    int nst, kt_w0, count;
    __device__ __forceinline__ int tile(int v) const { return v < nst ? v : kt_w0 + v - nst; }
};

__device__ __forceinline__ TileSpan tile_span(const KeyRows& r) {
    TileSpan t;
    t.kt_w0 = r.klo / kBK;
    const int kt_w1 = r.khi > r.klo ? (r.khi + kBK - 1) / kBK : t.kt_w0;
    // A sink tile that reaches the first window tile is that tile.
    const int nst = (r.sink_hi + kBK - 1) / kBK;
    t.nst = kt_w1 > t.kt_w0 ? min(nst, t.kt_w0) : nst;
    t.count = t.nst + (kt_w1 - t.kt_w0);
    return t;
}

// The key-tile indices (in tile_span order) of the tiles that some query at
// positions [pf, pl] sees within M of its position: a contiguous run
// [vb0, vb1), since tile_span's tiles rise with the index. Tiles before it lie
// M or more before every query, tiles after it M or more after.
__device__ __forceinline__ void band_tiles(const TileSpan& t, int pf, int pl, int M, int& vb0, int& vb1) {
    // Tiles below key tile x, in tile_span order.
    auto below = [&](int x) {
        const int sinks = min(t.nst, max(x, 0));
        const int win = min(max(x - t.kt_w0, 0), t.count - t.nst);
        return sinks + win;
    };
    // Far before every query: the tile's last key s with s - pf <= -M.
    const int kl = pf - M - (kBK - 1);  // key tile kt is far iff kt * kBK <= kl
    const int first_band = kl < 0 ? 0 : kl / kBK + 1;
    // Far after every query: the tile's first key s with s - pl >= M.
    const int kr = pl + M;              // key tile kt is far iff kt * kBK >= kr
    const int first_after = kr <= 0 ? 0 : (kr + kBK - 1) / kBK;
    vb0 = below(first_band);
    vb1 = max(vb0, below(first_after));
}

// Whether any / every query at positions [wpf, wpl] sees any / every key of
// [s_first, s_last] (every key also a loaded row).
__device__ __forceinline__ void tile_visibility(const Epilogue& e, int s_first, int s_last, int wpf,
                                                int wpl, const KeyRows& rows, bool& any_vis,
                                                bool& all_vis) {
    if (e.causal) {
        any_vis = s_first <= wpl && (e.window == 0 || s_last > wpf - e.window);
        all_vis = s_last <= wpf && (e.window == 0 || s_first > wpl - e.window);
    } else if (e.window > 0) {
        any_vis = (int64_t)s_first <= (int64_t)wpl + e.window && s_last >= wpf - e.window;
        all_vis = max(max(abs(wpf - s_first), abs(wpf - s_last)),
                      max(abs(wpl - s_first), abs(wpl - s_last))) <= e.window;
    } else {
        any_vis = true;
        all_vis = true;
    }
    all_vis = all_vis && s_first >= rows.klo && s_last < rows.khi;
    if (s_first < e.sinks) {
        // Sink keys: seen by every row (causal: at or before its position).
        any_vis = any_vis || !e.causal || s_first <= wpl;
        all_vis = all_vis || (s_last < rows.sink_hi && (!e.causal || s_last <= wpf));
    }
}

// Global -> registers -> LDS staging of the rows [kt*kBK, kt*kBK + kBK) of a
// K or V tile (width W floats, global row stride `stride`) by NT threads.
// A tile whose rows are all loaded rows (all but the first and last tiles of
// a range) is read straight: the tile's base is workgroup-uniform and each
// lane adds a fixed 32-bit byte offset. Elsewhere rows that are not loaded
// read a clamped, in-bounds row instead and are replaced by zeros, so the
// loads need no branches. stride <= 65536 heads x 256 floats, so an offset
// inside a tile (< kBK * stride * 4 bytes = 2^31) fits in 32 bits.
// The tile may be wider than the rows (WP >= W floats per LDS row, 80-wide
// rows in a 96-wide tile): columns past W are zeros and never read from
// memory.
template <int W, int NT, int WP = W>
__device__ __forceinline__ void fetch_rows(float4 (&st)[kBK * WP / 4 / NT], const float* base,
                                           int64_t stride, int kt, const KeyRows& rows) {
    const int s0 = kt * kBK;
    const bool whole = ((s0 >= rows.klo) & (s0 + kBK <= rows.khi)) | (s0 + kBK <= rows.sink_hi);
    if (whole) {
        const char* tb = reinterpret_cast<const char*>(base + (int64_t)s0 * stride);
#pragma unroll
        for (int j = 0; j < kBK * WP / 4 / NT; ++j) {
            const int f = (int)threadIdx.x + j * NT;
            const uint32_t row = (uint32_t)(f / (WP / 4)), c4 = (uint32_t)(f % (WP / 4));
            const uint32_t off = (row * (uint32_t)stride + 4u * c4) * 4u;
            if (WP == W || c4 < (uint32_t)(W / 4)) st[j] = *reinterpret_cast<const float4*>(tb + off);
            else st[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kBK * WP / 4 / NT; ++j) {
        const int f = (int)threadIdx.x + j * NT;
        const int row = f / (WP / 4), c4 = f % (WP / 4);
        const int s = s0 + row;
        const bool ok = rows.loaded(s) && (WP == W || c4 < W / 4);
        // The nearest row of [klo, khi) (khi - 1 when that range is empty):
        // usually a cache line the neighbouring loads touch anyway.
        const int sc = rows.loaded(s) ? s : min(max(s, rows.klo), rows.khi - 1);
        const float4 x = *reinterpret_cast<const float4*>(base + sc * stride + 4 * min(c4, W / 4 - 1));
        st[j].x = ok ? x.x : 0.0f;
        st[j].y = ok ? x.y : 0.0f;
        st[j].z = ok ? x.z : 0.0f;
        st[j].w = ok ? x.w : 0.0f;
    }
}

template <int W, int NT>
__device__ __forceinline__ void stage_rows(const float4 (&st)[kBK * W / 4 / NT], float* tile) {
#pragma unroll
    for (int j = 0; j < kBK * W / 4 / NT; ++j) {
        const int f = (int)threadIdx.x + j * NT;
        const int row = f / (W / 4), c4 = f % (W / 4);
        *reinterpret_cast<float4*>(tile + row * (W + kPad) + 4 * c4) = st[j];
    }
}

// The bucketed position bias through LDS: the distance -> bucket table
// (pb_dt bytes) and the weights of the workgroup's heads ([head][bucket]),
// filled once per workgroup, so that a score's term costs two LDS reads
// rather than two dependent memory loads (which inside the key loop also
// made the wave wait for every load issued before them, the next tile's K
// rows included). Bytes a kernel of up to nh_max heads per workgroup adds
// to its LDS when the term is on:
__host__ __device__ constexpr size_t pb_lds_bytes(int nh_max) {
    return ATTN_PB_MAX_DIST + sizeof(float) * (size_t)nh_max * 2 * ATTN_PB_MAX_BUCKETS;
}

// Fill the tables for heads h0 .. h0 + nh - 1 (all threads of the block take
// part; the caller's next barrier publishes them). Weights of local head hl
// start at w + hl * pb_nbk(e).
__device__ __forceinline__ int pb_nbk(const Epilogue& e) { return e.pb_bidir ? 2 * e.pb_n : e.pb_n; }
__device__ __forceinline__ void pb_fill(const Epilogue& e, uint8_t* bkt, float* w, int h0, int nh) {
    const int nt = (int)blockDim.x;
    for (int d = (int)threadIdx.x; d < e.pb_dt; d += nt) bkt[d] = e.pb_bucket[d];
    const int nbk = pb_nbk(e);
    for (int i = (int)threadIdx.x; i < nh * nbk; i += nt) {
        const int hl = i / nbk, b = i - hl * nbk;
        w[i] = e.pb_weight[b * e.pb_heads + h0 + hl];
    }
}

// position_bias with the tables in LDS (whead: the row's head's weights).
__device__ __forceinline__ float pb_lds(const Epilogue& e, const uint8_t* bkt, const float* whead, int pos, int s) {
    const int d = abs(pos - s);
    int b = d < e.pb_dt ? (int)bkt[d] : e.pb_n - 1;
    if (e.pb_bidir && s > pos) b += e.pb_n;
    return whead[b];
}

// Whether a tile's bias entries can come four at a time: the bias rows start
// 16-byte aligned when S is a multiple of 4 (the base pointer always is: the
// host refuses others).
__device__ __forceinline__ bool bias_vec4(const Problem& p) {
    return p.ep.bias_kind != ATTN_BIAS_NONE && (p.S & 3) == 0;
}

// The bias entries of (head h, query row t at position pos) for NQ groups of
// four keys, group j at s0 + j * step .. + 3 (s0 and step multiples of 4):
// the bias input's entry (one 128-bit load per group when `vec`, bias_vec4;
// else one per entry, clamped in bounds) plus, with pb_w the head's weights
// in LDS (NULL: off), the bucketed position bias; 0 without either. All
// groups' loads are requested under one branch, so they are in flight
// together. Past the last key (only in a tile's masked tail) the entries are
// those of the last keys.
template <int NQ>
__device__ __forceinline__ void bias_quads(const Problem& p, bool vec, int h, int t, int pos, int s0, int step,
                                           const uint8_t* pb_b, const float* pb_w, float (&b)[NQ][4]) {
    const int tc = min(t, (int)p.T - 1);
    const float* row = p.bias + (p.ep.bias_kind == ATTN_BIAS_HTS ? (int64_t)h * p.T + tc : (int64_t)tc) * p.S;
    if (vec) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(row + min(s0 + j * step, (int)p.S - 4));
            b[j][0] = v.x;
            b[j][1] = v.y;
            b[j][2] = v.z;
            b[j][3] = v.w;
        }
    } else if (p.ep.bias_kind != ATTN_BIAS_NONE) {
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) b[j][i] = row[min(max(s0 + j * step + i, 0), (int)p.S - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) b[j][i] = 0.0f;
    }
    if (pb_w) {
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) b[j][i] += pb_lds(p.ep, pb_b, pb_w, pos, s0 + j * step + i);
    }
}

template <typename K>
hipError_t set_lds_limit(K kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace pf
}  // namespace attn
