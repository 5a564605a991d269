// Prefill path of op `attention`: many query rows, flash-style, with both
// contractions on fp32 matrix cores (v_mfma_f32_32x32x2f32).
//
// A workgroup is 4 waves; each wave owns 32 query rows of one head, and the
// waves of a workgroup share one KV head (heads of the same group side by
// side, or consecutive query blocks of one head). K and V tiles of 32 key rows
// are staged in LDS, double-buffered, and read by all four waves. The next
// tile's K rows are fetched from global memory while QK^T runs and written to
// LDS after it; its V rows likewise around PV, so only one of the two is ever
// held in registers.
//
// Lane layouts of v_mfma_f32_32x32x2f32 (A 32x2, B 2x32, D 32x32, 64 lanes):
// A[i][k] sits in lane i + 32k, B[k][j] in lane j + 32k, and D[i][j] in lane
// j + 32*((i/4)%2), register 4*(i/8) + i%4.
//
// Scores are formed transposed, S^T = K Q^T, so a lane holds one query
// (column l%32) and 16 keys. That accumulator is then used as it stands as
// the B operand of O^T = V^T P^T: register r of lane l is P^T[key f(r, l/32)]
// [query l%32] with f(r, h) = 8(r/4) + 4h + r%4, and the V operand is read
// for exactly those keys. No score ever moves between lanes, and the score
// matrix never leaves registers.
//
// Contraction orders are chosen for wide LDS reads: in QK^T, k-step kk of
// half h uses d = h*D/2 + kk, so a lane reads D/2 consecutive floats of its
// key row (and holds the matching D/2 of its query row in registers); in PV,
// row i of output block b is dv = (DV/32) i + b, so a lane reads DV/32
// consecutive floats of a V row per k-step and writes DV/32 consecutive
// output floats per accumulator register.
//
// Online softmax per query in the base-2 domain with a lazily moved
// reference maximum (as in the decode path). Key tiles a workgroup cannot see
// are skipped; tiles that every query of a wave sees skip the mask. Rows of a
// tile outside the workgroup's visible key range are zero-filled, never read.
//
// When the grid would be too small to fill the chip (few query rows, as in
// chunked prefill), each workgroup's key range is split into `ksplit` parts;
// every part writes its unnormalised partial state to the workspace in the
// decode path's layout, and the decode combine kernel merges them.
//
// A 16x16x4 variant with 16 query rows per wave (prefill16.hip) serves wide
// heads; the host picks one per shape.
//
// Relative key/value embeddings (REL instances; the IR schema page's
// attention property relative_kv, read as Shaw et al.'s relative position
// representations): key s of query row t uses embedding row
// r = clip(s - pos, -M, M) + M, rel_k[r] joining k before the product with q
// and rel_v[r] joining v in the weighted sum. Per wave and key tile, with
// d = s - pos spanning [d_lo, d_lo + 62] over the wave's 32 queries:
//   - a tile whose d are all <= -M (or all >= M) uses row 0 (or 2M) for
//     every key: q . rel_k[0] is a per-query constant added to the scores,
//     and the tile's weight sum joins a per-query sum wL (or wR) that
//     multiplies rel_v[0] (or rel_v[2M]) once at the end (rescaled with the
//     running maximum like the softmax sum);
//   - any other tile (the band within M of the diagonal) forms q . rel_k for
//     the 64 relative rows d_lo .. d_lo + 63 on the matrix cores into the
//     wave's own LDS rows, adds entry d - d_lo to each score, and after the
//     softmax scatters the weights by d into the same rows for a second
//     contraction with the rel_v rows (O^T += rel_v^T P_rel^T).
// A wave's LDS rows are its own, and a wave's LDS accesses complete in
// order, so no barrier is needed around them.
#include "prefill_common.h"
#include "rope_device.h"

namespace attn {

namespace {

using namespace pf;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBQ = 32;  // query rows per wave

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// NB consecutive floats from LDS (NB = 2, 3 or a multiple of 4).
template <int NB>
__device__ __forceinline__ void lds_read(const float* src, float (&dst)[NB]) {
    if constexpr (NB == 3) {
        // 96-wide rows: three floats at a 12-byte stride, read one by one.
        dst[0] = src[0];
        dst[1] = src[1];
        dst[2] = src[2];
    } else if constexpr (NB % 4 == 0) {
#pragma unroll
        for (int b = 0; b < NB; b += 4) {
            const float4 w = *reinterpret_cast<const float4*>(src + b);
            dst[b] = w.x;
            dst[b + 1] = w.y;
            dst[b + 2] = w.z;
            dst[b + 3] = w.w;
        }
    } else {
        static_assert(NB == 2, "vHeadDim must be 64, 96 or a multiple of 128");
        const float2 w = *reinterpret_cast<const float2*>(src);
        dst[0] = w.x;
        dst[1] = w.y;
    }
}

// Waves per SIMD the register budget allows (two while q, o and staging fit
// in 256 registers per lane).
constexpr int prefill_min_waves(int D, int DV) { return D + DV <= 256 ? 2 : 1; }
// The same for the instances with relative key/value embeddings (their band
// tiles hold the relative rows' scores and weights as well): two only at 64/64.
constexpr int prefill_rel_waves(int D, int DV) { return D + DV <= 128 ? 2 : 1; }

constexpr int kRelRows = 64;  // relative rows per band tile: d_lo .. d_lo + 63

// Tile widths: the row widths rounded up to 32 floats (80-wide rows sit in
// 96-wide tiles whose last 16 columns are zeros, and q's are zeros there too).
constexpr int tile_width(int w) { return (w + 31) / 32 * 32; }

template <int D, int DV>
struct PrefillShape {
    static constexpr int DP = tile_width(D), DVP = tile_width(DV);
    static constexpr int KLD = DP + kPad;   // LDS row stride of a K tile
    static constexpr int VLD = DVP + kPad;  // LDS row stride of a V tile
    static constexpr int KF4 = kBK * DP / 4 / kThreads;   // float4 per thread per K tile
    static constexpr int VF4 = kBK * DVP / 4 / kThreads;  // float4 per thread per V tile
    static constexpr int NB = DVP / 32;     // output blocks (and V floats per lane per k-step)
    static constexpr size_t lds_bytes = sizeof(float) * 2 * kBK * (size_t)(KLD + VLD);
    // REL instances: each wave's [32 queries][kRelRows] rows after the tiles.
    static constexpr size_t rel_lds_bytes = sizeof(float) * kWaves * kBQ * kRelRows;
};

// RM: relative key/value embeddings. 0: off. 2: on, every tile (band tiles
// with their per-key rows). 1: on, for a launch of the tiles beyond the
// tables' reach for every row of the workgroup (Args::part 1): the band code
// is left out, so the instance needs no more registers than the epilogue one.
template <int D, int DV, bool EPI, int RM>
__global__ __launch_bounds__(kThreads, RM == 2 ? prefill_rel_waves(D, DV) : prefill_min_waves(D, DV)) void prefill_kernel(
    Problem p, Args a) {
    constexpr bool REL = RM != 0;
    constexpr bool BAND = RM == 2;
    using Sh = PrefillShape<D, DV>;
    constexpr int KLD = Sh::KLD, VLD = Sh::VLD, NB = Sh::NB, DP = Sh::DP, DVP = Sh::DVP;
    extern __shared__ float lds[];
    float* ktile = lds;                       // [2][kBK][KLD]
    float* vtile = lds + 2 * kBK * KLD;       // [2][kBK][VLD]

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int col = lane & 31;

    const int hpg = p.H / p.G;
    const int qsub = kWaves / a.nh;
    const Coords c = wg_coords(a);
    const int ks = c.ks, qb = c.qb, g = c.g, hgi = c.hgi;
    const int h = g * hpg + hgi * a.nh + wave % a.nh;
    const int qwg0 = qb * qsub * kBQ;                 // first query row of the workgroup
    const int q0 = qwg0 + (wave / a.nh) * kBQ;        // first query row of this wave
    const int T = (int)p.T, S = (int)p.S;
    const int t = q0 + col;                           // this lane's query row
    const bool trow = t < T;
    const int pos = p.ep.pos_offset + t;

    // This lane's half of its query row: q[t, h*D + half*DP/2 + kk], kk < DP/2
    // (zeros past D).
    float qreg[DP / 2];
    {
        const int tc = min(t, T - 1);
        const float* qhead = p.q + (int64_t)tc * p.H * D + (int64_t)h * D;
#pragma unroll
        for (int kk = 0; kk < DP / 2; kk += 4) {
            const int c = half * (DP / 2) + kk;
            const bool in = DP == D || c < D;
            // With a rotary embedding on q (rope.on is uniform), each channel is
            // turned as it is loaded.
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (in)
                v = p.rope.on ? rope_channels4(p.rope, qhead, c, p.rope.pos0 + tc)
                              : *reinterpret_cast<const float4*>(qhead + c);
            qreg[kk] = trow ? v.x : 0.0f;
            qreg[kk + 1] = trow ? v.y : 0.0f;
            qreg[kk + 2] = trow ? v.z : 0.0f;
            qreg[kk + 3] = trow ? v.w : 0.0f;
        }
    }

    // Keys any query row of the workgroup can see.
    const int wg_last = min(qwg0 + qsub * kBQ, T) - 1;
    int klo, khi;
    visible_keys(p.ep, S, p.ep.pos_offset + qwg0, p.ep.pos_offset + wg_last, klo, khi);
    // This wave's own query positions (for whole-tile visibility checks).
    const int wq_last = min(q0 + kBQ, T) - 1;
    const int wpf = p.ep.pos_offset + q0, wpl = p.ep.pos_offset + max(wq_last, q0);

    f32x16 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.0f;
    float m = -INFINITY, l = 0.0f;

    // Relative embeddings: this wave's LDS rows, the per-query products with
    // rows 0 and 2M, and the weight sums of the keys beyond reach.
    const int M = REL ? p.ep.rel_max : 0;
    float* wrel = lds + 2 * kBK * (KLD + VLD) + wave * (kBQ * kRelRows) + col * kRelRows;
    float qrel0 = 0.0f, qrelN = 0.0f, wL = 0.0f, wR = 0.0f;
    if constexpr (REL) {
        const float* r0 = p.ep.rel_k + half * (DP / 2);
        const float* rN = p.ep.rel_k + (int64_t)(2 * M) * D + half * (DP / 2);
        float a0 = 0.0f, aN = 0.0f;
#pragma unroll
        for (int kk = 0; kk < DP / 2; kk += 4) {
            if (DP != D && half * (DP / 2) + kk >= D) continue;  // q is zero there
            const float4 x0 = *reinterpret_cast<const float4*>(r0 + kk);
            const float4 xN = *reinterpret_cast<const float4*>(rN + kk);
            a0 = fmaf(qreg[kk], x0.x, fmaf(qreg[kk + 1], x0.y, fmaf(qreg[kk + 2], x0.z, fmaf(qreg[kk + 3], x0.w, a0))));
            aN = fmaf(qreg[kk], xN.x, fmaf(qreg[kk + 1], xN.y, fmaf(qreg[kk + 2], xN.z, fmaf(qreg[kk + 3], xN.w, aN))));
        }
        qrel0 = a0 + __shfl_xor(a0, 32, 64);
        qrelN = aN + __shfl_xor(aN, 32, 64);
    }

    // This workgroup's part of its key tiles (sink tiles, then window tiles):
    // with relative embeddings split over two launches, the tiles beyond
    // their reach (part 1, index j skipping the band run [vb0, vb1)) or the
    // band run alone (part 2).
    const KeyRows rows = key_rows(p.ep, klo, khi);
    const TileSpan span = tile_span(rows);
    int vb0 = 0, vb1 = 0;
    if (a.part != 0) band_tiles(span, p.ep.pos_offset + qwg0, p.ep.pos_offset + wg_last, M, vb0, vb1);
    const int nsel = a.part == 0 ? span.count : a.part == 1 ? span.count - (vb1 - vb0) : vb1 - vb0;
    const int skip = a.part == 1 ? vb1 - vb0 : 0;
    const int first = a.part == 2 ? vb0 : 0;
    auto tile_of = [&](int jj) {
        const int v = first + (jj < vb0 || a.part != 1 ? jj : jj + skip);
        return span.tile(v);
    };
    const int per = (nsel + a.ksplit - 1) / a.ksplit;
    const int v0 = min(nsel, ks * per);
    const int v1 = min(nsel, v0 + per);

    const int64_t kstride = (int64_t)p.G * D, vstride = (int64_t)p.G * DV;
    const float* kg = p.k + (int64_t)g * D;
    const float* vg = p.v + (int64_t)g * DV;
    float4 kst[Sh::KF4], vst[Sh::VF4];

    const float qk_scale = p.ep.scale * kLog2e;
    const float slope = alibi_slope(p.ep, h);
    const bool vec_bias = bias_vec4(p);
    // Bucketed position bias: its tables in LDS past the tiles (and the
    // relative rows), filled here and published by the loop's first barrier.
    const uint8_t* pb_b = nullptr;
    const float* pb_w = nullptr;
    if (EPI && p.ep.pb_weight) {
        uint8_t* b = reinterpret_cast<uint8_t*>(lds + 2 * kBK * (KLD + VLD) + (RM == 2 ? kWaves * kBQ * kRelRows : 0));
        float* w = reinterpret_cast<float*>(b + ATTN_PB_MAX_DIST);
        pb_fill(p.ep, b, w, g * hpg + hgi * a.nh, a.nh);
        pb_b = b;
        pb_w = w + (wave % a.nh) * pb_nbk(p.ep);
    }
    if (v0 < v1) {
        fetch_rows<D, kThreads, DP>(kst, kg, kstride, tile_of(v0), rows);
        fetch_rows<DV, kThreads, DVP>(vst, vg, vstride, tile_of(v0), rows);
        stage_rows<DP, kThreads>(kst, ktile);
        stage_rows<DVP, kThreads>(vst, vtile);
    }
    for (int v = v0; v < v1; ++v) {
        const int kt = tile_of(v);
        const int buf = (v - v0) & 1;
        const bool more = v + 1 < v1;
        const int kt_next = tile_of(v + 1);
        __syncthreads();  // tile `kt` is in LDS; everyone is done with the other buffer
        if constexpr (EPI) {
            if (more) fetch_rows<D, kThreads, DP>(kst, kg, kstride, kt_next, rows);
        }

        const int s_first = kt * kBK;
        bool any_vis, all_vis;
        tile_visibility(p.ep, s_first, s_first + kBK - 1, wpf, wpl, rows, any_vis, all_vis);
        // Whether the tile holds attention sinks (their rule is checked only then).
        const bool sink_tile = s_first < p.ep.sinks;

        const float* kt_ = ktile + buf * kBK * KLD;
        const float* vt_ = vtile + buf * kBK * VLD;
        float x[16];
        int rel_cls = 0, d_lo = 0, delta = 0;  // REL: 0 band tile, 1 every key at row 0, 2 every key at row 2M
        // Without epilogue terms the next tile's K rows go out here, after
        // the tile's visibility is worked out, not right after the barrier:
        // the Llama-shaped causal prefill measured 6% faster so (1084 against
        // 1154 us per call, three rounds on one box). With them (bias loads
        // ahead of the matrix work) the earlier issue was faster.
        if constexpr (!EPI) {
            if (more) fetch_rows<D, kThreads, DP>(kst, kg, kstride, kt_next, rows);
        }
        if (any_vis) {
            // Bias entries of the tile, requested before the matrix work so
            // that it hides their latency.
            float bpre[EPI ? 4 : 1][4];
            if constexpr (EPI) bias_quads<4>(p, vec_bias, h, t, pos, s_first + 4 * half, 8, pb_b, pb_w, bpre);
            // S^T = K Q^T for 32 keys x 32 queries.
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
            const float* krow = kt_ + col * KLD + half * (DP / 2);
#pragma unroll
            for (int kk = 0; kk < DP / 2; kk += 4) {
                const float4 kv = *reinterpret_cast<const float4*>(krow + kk);
                sacc = mfma32(kv.x, qreg[kk], sacc);
                sacc = mfma32(kv.y, qreg[kk + 1], sacc);
                sacc = mfma32(kv.z, qreg[kk + 2], sacc);
                sacc = mfma32(kv.w, qreg[kk + 3], sacc);
                // Keep the scheduler from hoisting every LDS read of the tile
                // at once (it would need DP/2 registers for them).
                if (kk % 16 == 12) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (REL) {
                // The relative-key term joins the product before the scale.
                d_lo = s_first - wpl;
                const int d_hi = s_first + kBK - 1 - wpf;
                rel_cls = d_hi <= -M ? 1 : (d_lo >= M || !BAND ? 2 : 0);
                if (rel_cls == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[r] += qrel0;
                } else if (rel_cls == 2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[r] += qrelN;
                } else if constexpr (BAND) {
                    // q . rel_k[clip(d) + M] for d = d_lo + i, i < 64 (rows
                    // i = 32 ps + col on the A side), into the wave's LDS rows.
#pragma unroll
                    for (int ps = 0; ps < kRelRows / 32; ++ps) {
                        const int rr = min(max(d_lo + 32 * ps + col, -M), M) + M;
                        const float* rk = p.ep.rel_k + (int64_t)rr * D + half * (DP / 2);
                        f32x16 racc;
#pragma unroll
                        for (int r = 0; r < 16; ++r) racc[r] = 0.0f;
#pragma unroll
                        for (int kk = 0; kk < DP / 2; kk += 4) {
                            const bool in = DP == D || half * (DP / 2) + kk < D;  // q is zero past D
                            const float4 kv = in ? *reinterpret_cast<const float4*>(rk + kk)
                                                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                            racc = mfma32(kv.x, qreg[kk], racc);
                            racc = mfma32(kv.y, qreg[kk + 1], racc);
                            racc = mfma32(kv.z, qreg[kk + 2], racc);
                            racc = mfma32(kv.w, qreg[kk + 3], racc);
                        }
#pragma unroll
                        for (int r = 0; r < 16; ++r) wrel[32 * ps + 8 * (r >> 2) + 4 * half + (r & 3)] = racc[r];
                    }
                    // Key f(r, half) of query pos sits at d - d_lo = f + (wpl - pos).
                    delta = min(max(wpl - pos, 0), kBK - 1);
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[r] += wrel[8 * (r >> 2) + 4 * half + (r & 3) + delta];
                }
            }

            // Score epilogue, then the mask; keys of register r: f(r, half).
            int sk[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sk[r] = s_first + 8 * (r >> 2) + 4 * half + (r & 3);
                x[r] = sacc[r];
            }
            if constexpr (EPI) {
                float bb[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) bb[r] = bpre[r >> 2][r & 3];
                score_epilogue_n<16>(x, p.ep, slope, pos, sk, bb);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] *= qk_scale;
            }
            if (!all_vis) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int s = sk[r];
                    bool vis = (s < rows.khi) & window_visible(p.ep, pos, s);
                    if (sink_tile) vis = vis | ((s < rows.khi) & sink_visible(p.ep, pos, s));
                    x[r] = vis ? x[r] : -INFINITY;
                }
            }
        }
        if (more) stage_rows<DP, kThreads>(kst, ktile + (buf ^ 1) * kBK * KLD);

        if (any_vis) {
            // Online softmax for this lane's query (both halves share the max).
            float mx = x[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            if (mx > m + kLazy) {
                const float alpha = fast_exp2(m - mx);
                l *= alpha;
                if constexpr (REL) {
                    wL *= alpha;
                    wR *= alpha;
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
                m = mx;
            }
            const float mu = m == -INFINITY ? 0.0f : m;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                x[r] = fast_exp2(x[r] - mu);
                ps += x[r];
            }
            l += ps;
            if constexpr (REL) {
                if (rel_cls == 1) {
                    wL += ps;
                } else if (rel_cls == 2) {
                    wR += ps;
                } else if (BAND && p.ep.rel_v) {
                    // The weights by relative offset (zero where no key of
                    // this query falls), then O^T += rel_v^T P_rel^T.
#pragma unroll
                    for (int e = 0; e < 32; e += 4)
                        *reinterpret_cast<float4*>(wrel + 32 * half + e) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                    for (int r = 0; r < 16; ++r) wrel[8 * (r >> 2) + 4 * half + (r & 3) + delta] = x[r];
#pragma unroll
                    for (int ps2 = 0; ps2 < kRelRows / 32; ++ps2) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int i = 32 * ps2 + 8 * (r >> 2) + 4 * half + (r & 3);
                            const int rr = min(max(d_lo + i, -M), M) + M;
                            float vv[NB];
                            const float* rv = p.ep.rel_v + (int64_t)rr * DV + NB * col;
#pragma unroll
                            for (int b = 0; b < NB; ++b) vv[b] = DVP == DV || NB * col + b < DV ? rv[b] : 0.0f;
                            const float pw = wrel[i];
#pragma unroll
                            for (int b = 0; b < NB; ++b) o[b] = mfma32(vv[b], pw, o[b]);
                        }
                    }
                }
            }
        }
        if (more) fetch_rows<DV, kThreads, DVP>(vst, vg, vstride, kt_next, rows);

        if (any_vis) {
            // O^T += V^T P^T: k-step r uses keys f(r, half) and P from register r.
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * half + (r & 3);
                float vv[NB];
                lds_read<NB>(vt_ + key * VLD + NB * col, vv);
#pragma unroll
                for (int b = 0; b < NB; ++b) o[b] = mfma32(vv[b], x[r], o[b]);
                if (NB * (r + 1) % 16 == 0) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (more) stage_rows<DVP, kThreads>(vst, vtile + (buf ^ 1) * kBK * VLD);
    }

    // Register r of block b is dv = NB*(8(r/4) + 4 half + r%4) + b.
    const float lt = l + __shfl_xor(l, 32, 64);
    if constexpr (REL) {
        // Keys beyond reach: their weight sums times rel_v[0] and rel_v[2M].
        const float wLt = wL + __shfl_xor(wL, 32, 64), wRt = wR + __shfl_xor(wR, 32, 64);
        if (p.ep.rel_v) {
            const float* v0 = p.ep.rel_v;
            const float* vN = p.ep.rel_v + (int64_t)(2 * M) * DV;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (DVP == DV || NB * i + b < DV)
                        o[b][r] = fmaf(wLt, v0[NB * i + b], fmaf(wRt, vN[NB * i + b], o[b][r]));
            }
        }
    }
    if (!trow) return;
    const int64_t th = (int64_t)t * p.H + h;
    float* dst;
    float sc;
    if (a.kslots == 1) {
        dst = p.out + th * DV;
        sc = lt > 0.0f ? 1.0f / lt : 0.0f;
    } else {
        // Unnormalised partial state (max in the base-2 domain, sum, acc).
        const int slot = a.kslot0 + ks;
        dst = a.ws + (th * a.kslots + slot) * DV;
        sc = 1.0f;
        if (half == 0) {
            float* ml = a.ws + (int64_t)T * p.H * a.kslots * DV + (th * a.kslots + slot) * 2;
            ml[0] = m;
            ml[1] = lt;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * half + (r & 3);
        if constexpr (NB % 4 == 0) {
#pragma unroll
            for (int b = 0; b < NB; b += 4)
                *reinterpret_cast<float4*>(dst + NB * i + b) =
                    make_float4(o[b][r] * sc, o[b + 1][r] * sc, o[b + 2][r] * sc, o[b + 3][r] * sc);
        } else if constexpr (NB == 3) {
#pragma unroll
            for (int b = 0; b < 3; ++b)
                if (DVP == DV || 3 * i + b < DV) dst[3 * i + b] = o[b][r] * sc;
        } else {
            *reinterpret_cast<float2*>(dst + NB * i) = make_float2(o[0][r] * sc, o[1][r] * sc);
        }
    }
}

template <int D, int DV, bool EPI, int RM = 0>
hipError_t launch_t(const Problem& p, const Args& a, const Launch& L) {
    auto kern = prefill_kernel<D, DV, EPI, RM>;
    constexpr size_t lds = PrefillShape<D, DV>::lds_bytes + (RM == 2 ? PrefillShape<D, DV>::rel_lds_bytes : 0);
    constexpr size_t lds_pb = EPI ? pb_lds_bytes(kWaves) : 0;  // with the bucketed position bias
    static bool configured = false;
    if (!configured) {
        const hipError_t e = set_lds_limit(kern, lds + lds_pb);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int64_t nwg = (int64_t)a.qblocks * p.G * a.hgroups * a.ksplit;
    const size_t bytes = lds + (p.ep.pb_weight ? lds_pb : 0);
    return launch_kernel(kern, dim3((unsigned)nwg), dim3(kThreads), (uint32_t)bytes, L, p, a);
}

template <int D, int DV>
hipError_t launch_dims(const Problem& p, const Args& a, const Launch& L) {
    if (p.ep.rel_k) {
        if constexpr (D + DV <= 256) {
            if constexpr (D + DV > 128) {
                // The far tiles need the epilogue instance only for terms
                // besides the embeddings (their per-row constant joins the
                // product before the scale either way).
                const bool other = p.ep.softcap > 0.0f || p.ep.has_alibi || p.ep.bias_kind != ATTN_BIAS_NONE ||
                                   p.ep.pb_weight != nullptr;
                if (a.part == 1) return other ? launch_t<D, DV, true, 1>(p, a, L) : launch_t<D, DV, false, 1>(p, a, L);
            }
            return a.part == 1 ? hipErrorInvalidValue : launch_t<D, DV, true, 2>(p, a, L);
        }
        return hipErrorInvalidValue;
    }
    if (a.part != 0) return hipErrorInvalidValue;
    const bool epi = p.ep.any();
    return epi ? launch_t<D, DV, true>(p, a, L) : launch_t<D, DV, false>(p, a, L);
}

}  // namespace

hipError_t launch_prefill16(const Problem& p, const pf::Args& a, const Launch& L);

bool prefill_supported(int D, int Dv) {
    return (D == 64 && Dv == 64) || (D == 80 && Dv == 80) || (D == 96 && Dv == 96) || (D == 128 && Dv == 128) ||
           (D == 192 && Dv == 128) || (D == 256 && Dv == 256);
}

// Workgroups per CU the prefill kernels reach (registers and LDS).
int prefill_wgs_per_cu(int variant, int D, int Dv, bool rel) {
    if (variant == 16) return D + Dv <= 256 ? 2 : 1;
    return rel ? prefill_rel_waves(D, Dv) : prefill_min_waves(D, Dv);
}

// Relative key/value embeddings have 32x32x2 instances up to D + Dv = 256.
bool prefill_rel_supported(int D, int Dv) { return prefill_supported(D, Dv) && D + Dv <= 256; }

hipError_t launch_prefill(const Problem& p, const PrefillPlan& plan, float* ws, int part, const Launch& L) {
    Args a;
    a.nh = plan.nh;
    a.hgroups = (p.H / p.G) / plan.nh;
    a.qblocks = plan.qblocks;
    a.causal_order = p.ep.causal ? 1 : 0;
    a.ws = ws;
    a.part = part;
    a.kslots = plan.ksplit + plan.rel_band;
    a.ksplit = part == 2 ? plan.rel_band : plan.ksplit;
    a.kslot0 = part == 2 ? plan.ksplit : 0;
    if (part < 0 || part > 2 || (part != 0) != (plan.rel_band != 0) || (part != 0 && !p.ep.rel_k))
        return hipErrorInvalidValue;
    if (a.nh < 1 || a.hgroups < 1 || a.qblocks < 1 || a.ksplit < 1) return hipErrorInvalidValue;
    if (a.kslots > 1 && !ws) return hipErrorInvalidValue;
    if ((int64_t)a.qblocks * p.G * a.hgroups * a.ksplit > INT32_MAX) return hipErrorInvalidValue;
    if (plan.variant == 16) return part == 0 ? launch_prefill16(p, a, L) : hipErrorInvalidValue;
    if (plan.variant != 32) return hipErrorInvalidValue;
    if (p.D == 64 && p.Dv == 64) return launch_dims<64, 64>(p, a, L);
    if (p.D == 80 && p.Dv == 80) return launch_dims<80, 80>(p, a, L);
    if (p.D == 96 && p.Dv == 96) return launch_dims<96, 96>(p, a, L);
    if (p.D == 128 && p.Dv == 128) return launch_dims<128, 128>(p, a, L);
    if (p.D == 192 && p.Dv == 128) return launch_dims<192, 128>(p, a, L);
    if (p.D == 256 && p.Dv == 256) return launch_dims<256, 256>(p, a, L);
    return hipErrorInvalidValue;
}

}  // namespace attn
