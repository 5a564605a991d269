// Prefill path of op `attention`, 16x16x4 variant: 8 waves of 16 query rows,
// both contractions on v_mfma_f32_16x16x4f32.
//
// The same flash scheme as the 32x32x2 kernel (prefill.hip), with half the
// query rows per wave: q and the output accumulator then take D/4 and DV/4
// registers per lane instead of D/2 and DV/2, so wide heads (D = 192, 256)
// still fit two waves per SIMD, and each wave's softmax work hides under the
// other wave's matrix instructions.
//
// Lane layouts of v_mfma_f32_16x16x4f32 (A 16x4, B 4x16, D 16x16, 64 lanes):
// A[i][k] sits in lane i + 16k, B[k][j] in lane j + 16k, and D[i][j] in lane
// j + 16*(i/4), register i%4.
//
// Scores are formed transposed, S^T = K Q^T, in two 16-key blocks per 32-key
// tile: register r of lane l holds P^T[key 16kb + 4(l/16) + r][query l%16],
// which is exactly the B operand of O^T = V^T P^T for k-step (kb, r). In QK^T
// the lanes of quarter w = l/16 contract d = w*D/4 + kk, so a lane reads D/4
// consecutive floats of its key row. In PV, output block b holds
// dv = 64*(b/4) + 4i + b%4 for row i: the V operand of a lane is four
// float4s, 64 floats apart, so the 16 lanes of a quarter read 256 contiguous
// bytes per LDS instruction (no bank conflicts), and each accumulator
// register maps to float4 output stores.
#include "prefill_common.h"
#include "rope_device.h"

namespace attn {

namespace {

using namespace pf;

constexpr int kThreads16 = 512;
constexpr int kWaves16 = 8;
constexpr int kBQ16 = 16;  // query rows per wave

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, int DV>
struct Shape16 {
    static constexpr int KLD = D + kPad;
    static constexpr int VLD = DV + kPad;
    static constexpr int KF4 = kBK * D / 4 / kThreads16;
    static constexpr int VF4 = kBK * DV / 4 / kThreads16;
    static constexpr int NB = DV / 16;  // output blocks of 16 dv rows
    static constexpr size_t lds_bytes = sizeof(float) * 2 * kBK * (size_t)(KLD + VLD);
    static_assert(D % 64 == 0 && DV % 64 == 0, "head widths must be multiples of 64");
};

template <int D, int DV, bool EPI>
__global__ __launch_bounds__(kThreads16, 1) void prefill16_kernel(Problem p, Args a) {
    using Sh = Shape16<D, DV>;
    constexpr int KLD = Sh::KLD, VLD = Sh::VLD, NB = Sh::NB;
    extern __shared__ float lds[];
    float* ktile = lds;                  // [2][kBK][KLD]
    float* vtile = lds + 2 * kBK * KLD;  // [2][kBK][VLD]

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane >> 4;
    const int col = lane & 15;

    const int hpg = p.H / p.G;
    const int qsub = kWaves16 / a.nh;
    const Coords c = wg_coords(a);
    const int h = c.g * hpg + c.hgi * a.nh + wave % a.nh;
    const int qwg0 = c.qb * qsub * kBQ16;
    const int q0 = qwg0 + (wave / a.nh) * kBQ16;
    const int T = (int)p.T, S = (int)p.S;
    const int t = q0 + col;
    const bool trow = t < T;
    const int pos = p.ep.pos_offset + t;

    // This lane's quarter of its query row: q[t, h*D + quad*D/4 + kk], kk < D/4.
    float qreg[D / 4];
    {
        const int tc = min(t, T - 1);
        const float* qhead = p.q + (int64_t)tc * p.H * D + (int64_t)h * D;
#pragma unroll
        for (int kk = 0; kk < D / 4; kk += 4) {
            const float4 v = p.rope.on ? rope_channels4(p.rope, qhead, quad * (D / 4) + kk, p.rope.pos0 + tc)
                                       : *reinterpret_cast<const float4*>(qhead + quad * (D / 4) + kk);
            qreg[kk] = trow ? v.x : 0.0f;
            qreg[kk + 1] = trow ? v.y : 0.0f;
            qreg[kk + 2] = trow ? v.z : 0.0f;
            qreg[kk + 3] = trow ? v.w : 0.0f;
        }
    }

    const int wg_last = min(qwg0 + qsub * kBQ16, T) - 1;
    int klo, khi;
    visible_keys(p.ep, S, p.ep.pos_offset + qwg0, p.ep.pos_offset + wg_last, klo, khi);
    const int wq_last = min(q0 + kBQ16, T) - 1;
    const int wpf = p.ep.pos_offset + q0, wpl = p.ep.pos_offset + max(wq_last, q0);

    f32x4v o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f;

    // This workgroup's part of its key tiles (sink tiles, then window tiles).
    const KeyRows rows = key_rows(p.ep, klo, khi);
    const TileSpan span = tile_span(rows);
    const int per = (span.count + a.ksplit - 1) / a.ksplit;
    const int v0 = min(span.count, c.ks * per);
    const int v1 = min(span.count, v0 + per);

    const int64_t kstride = (int64_t)p.G * D, vstride = (int64_t)p.G * DV;
    const float* kg = p.k + (int64_t)c.g * D;
    const float* vg = p.v + (int64_t)c.g * DV;
    float4 kst[Sh::KF4], vst[Sh::VF4];
    const float qk_scale = p.ep.scale * kLog2e;
    const float slope = alibi_slope(p.ep, h);
    const bool vec_bias = bias_vec4(p);
    // Bucketed position bias: its tables in LDS past the tiles, filled here
    // and published by the loop's first barrier.
    const uint8_t* pb_b = nullptr;
    const float* pb_w = nullptr;
    if (EPI && p.ep.pb_weight) {
        uint8_t* b = reinterpret_cast<uint8_t*>(lds + 2 * kBK * (KLD + VLD));
        float* w = reinterpret_cast<float*>(b + ATTN_PB_MAX_DIST);
        pb_fill(p.ep, b, w, c.g * hpg + c.hgi * a.nh, a.nh);
        pb_b = b;
        pb_w = w + (wave % a.nh) * pb_nbk(p.ep);
    }

    if (v0 < v1) {
        fetch_rows<D, kThreads16>(kst, kg, kstride, span.tile(v0), rows);
        fetch_rows<DV, kThreads16>(vst, vg, vstride, span.tile(v0), rows);
        stage_rows<D, kThreads16>(kst, ktile);
        stage_rows<DV, kThreads16>(vst, vtile);
    }
    for (int v = v0; v < v1; ++v) {
        const int kt = span.tile(v);
        const int buf = (v - v0) & 1;
        const bool more = v + 1 < v1;
        const int kt_next = span.tile(v + 1);
        __syncthreads();  // tile `kt` is in LDS; everyone is done with the other buffer
        if (more) fetch_rows<D, kThreads16>(kst, kg, kstride, kt_next, rows);

        const int s_first = kt * kBK;
        bool any_vis, all_vis;
        tile_visibility(p.ep, s_first, s_first + kBK - 1, wpf, wpl, rows, any_vis, all_vis);
        // Whether the tile holds attention sinks (their rule is checked only then).
        const bool sink_tile = s_first < p.ep.sinks;

        const float* kt_ = ktile + buf * kBK * KLD;
        const float* vt_ = vtile + buf * kBK * VLD;
        float x[2][4];
        if (any_vis) {
            // Bias entries of the tile, requested before the matrix work so
            // that it hides their latency.
            float bpre[2][EPI ? 4 : 1];
            if constexpr (EPI) bias_quads<2>(p, vec_bias, h, t, pos, s_first + 4 * quad, 16, pb_b, pb_w, bpre);
            // Scores of both 16-key blocks, then the epilogue over the 8 scores
            // of the lane, then the mask. Score 4 kb + r: key s_first + 16 kb +
            // 4 quad + r.
            float xe[8];
            int sk[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4v sacc = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
                const float* krow = kt_ + (kb * 16 + col) * KLD + quad * (D / 4);
#pragma unroll
                for (int kk = 0; kk < D / 4; kk += 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(krow + kk);
                    sacc = mfma16(kv.x, qreg[kk], sacc);
                    sacc = mfma16(kv.y, qreg[kk + 1], sacc);
                    sacc = mfma16(kv.z, qreg[kk + 2], sacc);
                    sacc = mfma16(kv.w, qreg[kk + 3], sacc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xe[4 * kb + r] = sacc[r];
                    sk[4 * kb + r] = s_first + kb * 16 + 4 * quad + r;
                }
            }
            if constexpr (EPI) {
                float bb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) bb[i] = bpre[i >> 2][i & 3];
                score_epilogue_n<8>(xe, p.ep, slope, pos, sk, bb);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xe[i] *= qk_scale;
            }
            if (!all_vis) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = sk[i];
                    bool vis = (s < rows.khi) & window_visible(p.ep, pos, s);
                    if (sink_tile) vis = vis | ((s < rows.khi) & sink_visible(p.ep, pos, s));
                    xe[i] = vis ? xe[i] : -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i >> 2][i & 3] = xe[i];
        }
        if (more) stage_rows<D, kThreads16>(kst, ktile + (buf ^ 1) * kBK * KLD);

        if (any_vis) {
            // The four quarters of a lane column hold the same query.
            float mx = x[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            if (mx > m + kLazy) {
                const float alpha = fast_exp2(m - mx);
                l *= alpha;
#pragma unroll
                for (int b = 0; b < NB; ++b) o[b] *= alpha;
                m = mx;
            }
            const float mu = m == -INFINITY ? 0.0f : m;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[kb][r] = fast_exp2(x[kb][r] - mu);
                    l += x[kb][r];
                }
        }
        if (more) fetch_rows<DV, kThreads16>(vst, vg, vstride, kt_next, rows);

        if (any_vis) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float* vrow = vt_ + (kb * 16 + 4 * quad + r) * VLD + 4 * col;
                    float vv[NB];
#pragma unroll
                    for (int j = 0; j < NB / 4; ++j) {
                        const float4 w = *reinterpret_cast<const float4*>(vrow + 64 * j);
                        vv[4 * j] = w.x;
                        vv[4 * j + 1] = w.y;
                        vv[4 * j + 2] = w.z;
                        vv[4 * j + 3] = w.w;
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) o[b] = mfma16(vv[b], x[kb][r], o[b]);
                }
        }
        if (more) stage_rows<DV, kThreads16>(vst, vtile + (buf ^ 1) * kBK * VLD);
    }

    float lt = l + __shfl_xor(l, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (!trow) return;
    const int64_t th = (int64_t)t * p.H + h;
    float* dst;
    float sc;
    if (a.kslots == 1) {
        dst = p.out + th * DV;
        sc = lt > 0.0f ? 1.0f / lt : 0.0f;
    } else {
        const int slot = a.kslot0 + c.ks;
        dst = a.ws + (th * a.kslots + slot) * DV;
        sc = 1.0f;
        if (quad == 0) {
            float* ml = a.ws + (int64_t)T * p.H * a.kslots * DV + (th * a.kslots + slot) * 2;
            ml[0] = m;
            ml[1] = lt;
        }
    }
    // Register r of block b is row i = 4*quad + r: dv = 64*(b/4) + 4i + b%4.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 4 * quad + r;
#pragma unroll
        for (int j = 0; j < NB / 4; ++j)
            *reinterpret_cast<float4*>(dst + 64 * j + 4 * i) =
                make_float4(o[4 * j][r] * sc, o[4 * j + 1][r] * sc, o[4 * j + 2][r] * sc,
                            o[4 * j + 3][r] * sc);
    }
}

template <int D, int DV, bool EPI>
hipError_t launch16_t(const Problem& p, const Args& a, const Launch& L) {
    auto kern = prefill16_kernel<D, DV, EPI>;
    constexpr size_t lds = Shape16<D, DV>::lds_bytes;
    constexpr size_t lds_pb = EPI ? pb_lds_bytes(kWaves16) : 0;  // with the bucketed position bias
    static bool configured = false;
    if (!configured) {
        const hipError_t e = set_lds_limit(kern, lds + lds_pb);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int64_t nwg = (int64_t)a.qblocks * p.G * a.hgroups * a.ksplit;
    const size_t bytes = lds + (p.ep.pb_weight ? lds_pb : 0);
    return launch_kernel(kern, dim3((unsigned)nwg), dim3(kThreads16), (uint32_t)bytes, L, p, a);
}

template <int D, int DV>
hipError_t launch16_dims(const Problem& p, const Args& a, const Launch& L) {
    const bool epi = p.ep.any();
    return epi ? launch16_t<D, DV, true>(p, a, L) : launch16_t<D, DV, false>(p, a, L);
}

}  // namespace

hipError_t launch_prefill16(const Problem& p, const pf::Args& a, const Launch& L) {
    if (p.D == 64 && p.Dv == 64) return launch16_dims<64, 64>(p, a, L);
    if (p.D == 128 && p.Dv == 128) return launch16_dims<128, 128>(p, a, L);
    if (p.D == 192 && p.Dv == 128) return launch16_dims<192, 128>(p, a, L);
    if (p.D == 256 && p.Dv == 256) return launch16_dims<256, 256>(p, a, L);
    return hipErrorInvalidValue;
}

}  // namespace attn
