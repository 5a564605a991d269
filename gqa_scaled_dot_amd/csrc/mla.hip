// Latent (MLA) attention in absorbed form (the IR schema's op_mla_attention,
// read as DeepSeek-V2's multi-head latent attention).
//
// Head h attends with keys [k_b[h] c_s ; k_pe_s] and values v_b[h] c_s over
// the latent state rows [c_s | k_pe_s]. Associativity moves the
// up-projections off the key axis:
//   q_abs[t,h] = [k_b[h]^T q_nope[t,h] ; q_pe[t,h]]          (mla_absorb)
//   score(s)   = scale * q_abs[t,h] . state[s]                (mla_split)
//   o_lat      = softmax-weighted sum of c_s                  (mla_split)
//   out[t,h]   = v_b[h] o_lat                                 (mla_combine)
// so each latent row (R + P floats) is read once for every head and query
// row, instead of heads x (qk_nope + qk_rope + v_head_dim) floats of
// materialized keys and values.
//
// mla_split is a flash-decoding kernel on the matrix cores: all T*H rows
// share the single latent "KV head", so a workgroup takes one or two groups
// of 16 rows and a key chunk, stages 16- or 32-key tiles of the state in LDS
// (double-buffered), and the four waves of a row group split the channels: for scores wave w contracts R/4 latent
// channels and P/4 rotary channels (partial scores summed through LDS); for
// the weighted sum it owns the output channels [w R/4, (w+1) R/4). Scores
// are formed transposed (S^T = C Q^T with v_mfma_f32_16x16x4f32, keys on the
// A side), so register r of lane l holds the weight of key 4(l/16) + r for
// row l%16: exactly the B operand of O^T = C^T P^T, as in the prefill
// kernels. Partial (max, sum, acc) states of the key splits go to the
// workspace; mla_combine merges them and applies v_b.
//
// Lane layouts of v_mfma_f32_16x16x4f32 (A 16x4, B 4x16, D 16x16, 64 lanes):
// A[i][k] sits in lane i + 16k, B[k][j] in lane j + 16k, and D[i][j] in lane
// j + 16*(i/4), register i%4.
#include "device_common.h"

namespace attn {

namespace {

constexpr int kMlaThreads = 256;
constexpr int kMlaWaves = 4;
constexpr int kMlaKT = 16;   // keys per tile
constexpr int kMlaRB = 16;   // rows per workgroup
constexpr float kMlaLazy = 8.0f;
constexpr int kMlaMaxSplits = 1024;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mla_mfma(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// RG row groups of 16 rows share a workgroup (4 waves per group) and every
// key tile, which holds 16 * RG keys: with many rows (the 128-head shape)
// each staged tile then feeds twice the matrix work, and each barrier and
// tile load is paid half as often per instruction.
template <int R, int P, int RG>
struct MlaShape {
    static constexpr int DL = R + P;                            // latent row width
    static constexpr int NT = kMlaThreads * RG;                 // threads
    static constexpr int KT = kMlaKT * RG;                      // keys per tile
    static constexpr int NKB = KT / 16;                         // 16-key blocks per tile
    static constexpr int NQ = R / kMlaWaves / 4;                // latent channels per quad of a wave
    static constexpr int PQ = P / kMlaWaves / 4;                // rotary channels per quad of a wave
    static constexpr int KQ = NQ + PQ;                          // score k-steps per wave and 16 keys
    static constexpr int VW = R / kMlaWaves;                    // output channels per wave
    static constexpr int VG = VW / 64;                          // 64-channel groups per wave
    static constexpr int NB = VW / 16;                          // output blocks of 16 channels
    static constexpr int F4 = KT * DL / 4 / NT;                 // staging float4s per thread
    static constexpr size_t lds_bytes =
        sizeof(float) * (2 * KT * DL) + sizeof(f32x4v) * kMlaWaves * RG * NKB * 64;
    static_assert(R % 256 == 0 && P % 64 == 0, "R must be a multiple of 256, P of 64");
    static_assert(DL % 64 == 0, "rows must be whole 16-float4 bank groups for the swizzle");
    static_assert((KT * DL / 4) % NT == 0, "tile must split evenly over the threads");
    static_assert(lds_bytes <= 160 * 1024, "LDS");
};

// LDS tiles hold state rows unpadded (DL floats) with the float4 column c4 of
// row r stored at c4 ^ (r & 15): the 16 rows a score read touches at one
// column, and the 16 columns a weighted-sum read touches in one row, each
// fall on 16 different float4 bank groups (64 banks x 4 bytes = 16 float4s).
template <int DL>
__device__ __forceinline__ const float* tile_at(const float* tile, int r, int c4) {
    return tile + r * DL + 4 * (c4 ^ (r & 15));
}

// The latent/rotary channel that lane quad q of wave w contracts at score
// k-step kk: its quarter of the wave's latent channels, then of its rotary ones.
template <int R, int P>
__device__ __forceinline__ int score_channel(int w, int q, int kk) {
    constexpr int NQ = R / kMlaWaves / 4, PQ = P / kMlaWaves / 4;
    return kk < NQ ? w * (R / kMlaWaves) + q * NQ + kk : R + w * (P / kMlaWaves) + q * PQ + (kk - NQ);
}

// grid (splits, ceil(row_blocks / RG)), 256 * RG threads.
template <int R, int P, int RG>
__global__ __launch_bounds__(kMlaThreads * RG, 2 / RG) void mla_split_kernel(MlaProblem p, MlaPlan plan) {
    using Sh = MlaShape<R, P, RG>;
    constexpr int DL = Sh::DL, KQ = Sh::KQ, NB = Sh::NB, VG = Sh::VG, F4 = Sh::F4;
    constexpr int NT = Sh::NT, KT = Sh::KT, NKB = Sh::NKB;
    extern __shared__ __align__(16) float lds[];
    float* tiles = lds;                                                // [2][KT][DL], swizzled
    f32x4v* s_part = reinterpret_cast<f32x4v*>(lds + 2 * KT * DL);     // [RG*4 waves][NKB][64]

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int grp = wave / kMlaWaves;   // row group
    const int wv = wave % kMlaWaves;    // the wave's channel quarter
    const int lane = tid & 63;
    const int quad = lane >> 4;
    const int col = lane & 15;
    const int sp = blockIdx.x;
    const int nrows = (int)p.T * p.H;
    const int row = (blockIdx.y * RG + grp) * kMlaRB + col;  // this lane's (t, h) row
    const bool live = row < nrows;
    const int pos = p.vis.pos_offset + (live ? row / p.H : 0);

    // This split's keys: a chunk of the window range, or (the last split,
    // with attention sinks) the sink keys below it.
    const bool sink_split = plan.sink_hi > 0 && sp == (int)gridDim.x - 1;
    const int k0 = sink_split ? 0 : (int)(plan.range.lo + (int64_t)sp * plan.chunk);
    const int k1 = sink_split ? plan.sink_hi : (int)min(plan.range.hi, (int64_t)k0 + plan.chunk);
    const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;

    // q_abs of this lane's row, at the channels its quad contracts.
    float qreg[KQ];
    {
        const float* qrow = p.q_abs + (int64_t)(live ? row : 0) * DL;
#pragma unroll
        for (int kk = 0; kk < KQ; kk += 4) {
            const float4 v = *reinterpret_cast<const float4*>(qrow + score_channel<R, P>(wv, quad, kk));
            qreg[kk] = live ? v.x : 0.0f;
            qreg[kk + 1] = live ? v.y : 0.0f;
            qreg[kk + 2] = live ? v.z : 0.0f;
            qreg[kk + 3] = live ? v.w : 0.0f;
        }
    }

    // Global -> registers: KT state rows from key s0. Rows at or past k1 read
    // row k1 - 1 (in bounds) and are zeroed; a tile inside [k0, k1) reads
    // straight from a uniform base with fixed per-lane 32-bit offsets.
    float4 st[F4];
    auto fetch = [&](int s0) {
        if (s0 + KT <= k1) {
            const float* tb = p.state + (int64_t)s0 * DL;
#pragma unroll
            for (int j = 0; j < F4; ++j) {
                const uint32_t f = (uint32_t)tid + (uint32_t)j * NT;
                const uint32_t r = f / (DL / 4), c4 = f % (DL / 4);
                st[j] = *reinterpret_cast<const float4*>(tb + r * (uint32_t)DL + 4u * c4);
            }
        } else {
#pragma unroll
            for (int j = 0; j < F4; ++j) {
                const int f = tid + j * NT;
                const int r = f / (DL / 4), c4 = f % (DL / 4);
                const int s = s0 + r;
                const bool ok = s < k1;
                const float4 x =
                    *reinterpret_cast<const float4*>(p.state + (int64_t)(ok ? s : k1 - 1) * DL + 4 * c4);
                st[j] = ok ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    };
    auto stage = [&](int buf) {
        float* t = tiles + buf * KT * DL;
#pragma unroll
        for (int j = 0; j < F4; ++j) {
            const int f = tid + j * NT;
            const int r = f / (DL / 4), c4 = f % (DL / 4);
            *reinterpret_cast<float4*>(t + r * DL + 4 * (c4 ^ (r & 15))) = st[j];
        }
    };

    f32x4v o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f;

    if (ntiles > 0) {
        fetch(k0);
        stage(0);
    }
    for (int n = 0; n < ntiles; ++n) {
        const int buf = n & 1;
        const int s0 = k0 + n * KT;
        const bool more = n + 1 < ntiles;
        __syncthreads();  // tile n is in LDS; every wave is done with the other buffer and s_part
        if (more) fetch(s0 + KT);
        const float* tile = tiles + buf * KT * DL;
        // Let the scheduler interleave the tile's LDS reads with the matrix
        // instructions (V3-shaped split 106.5-106.7 us against 109.9-110.5).
        __builtin_amdgcn_iglp_opt(0);

        // Partial S^T over this wave's channels, per 16-key block kb: key
        // 16kb + col of the tile against this lane's row.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x4v sacc[3] = {f32x4v{0.0f, 0.0f, 0.0f, 0.0f}, f32x4v{0.0f, 0.0f, 0.0f, 0.0f},
                              f32x4v{0.0f, 0.0f, 0.0f, 0.0f}};
            const int kr = 16 * kb + col;
#pragma unroll
            for (int kk = 0; kk < KQ; kk += 4) {
                const float4 kv = *reinterpret_cast<const float4*>(
                    tile_at<DL>(tile, kr, score_channel<R, P>(wv, quad, kk) / 4));
                f32x4v& acc = sacc[(kk / 4) % 3];
                acc = mla_mfma(kv.x, qreg[kk], acc);
                acc = mla_mfma(kv.y, qreg[kk + 1], acc);
                acc = mla_mfma(kv.z, qreg[kk + 2], acc);
                acc = mla_mfma(kv.w, qreg[kk + 3], acc);
            }
            s_part[(wave * NKB + kb) * 64 + lane] = sacc[0] + sacc[1] + sacc[2];
        }
        __syncthreads();

        // Register r of block kb: key s0 + 16kb + 4*quad + r, row `row`. The
        // group's four partial sums, the mask, then the online softmax in
        // the base-2 domain with a lazily moved maximum.
        float x[NKB][4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x4v sc = s_part[((grp * kMlaWaves) * NKB + kb) * 64 + lane];
#pragma unroll
            for (int w = 1; w < kMlaWaves; ++w) sc += s_part[((grp * kMlaWaves + w) * NKB + kb) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + 16 * kb + 4 * quad + r;
                const bool vis = live & (s < k1) & key_visible(p.vis, pos, s);
                x[kb][r] = vis ? sc[r] * p.qk_scale : -INFINITY;
            }
        }
        float mx = x[0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (mx > m + kMlaLazy) {
            const float alpha = fast_exp2(m - mx);
            l *= alpha;
#pragma unroll
            for (int b = 0; b < NB; ++b) o[b] *= alpha;
            m = mx;
        }
        const float mu = m == -INFINITY ? 0.0f : m;
        float pr[NKB][4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[kb][r] = fast_exp2(x[kb][r] - mu);
                l += pr[kb][r];
            }

        // O^T += C^T P^T over this wave's output channels: k-step (kb, r)
        // takes keys 16kb + 4*quad + r; block 4g + u holds channel
        // wv*VW + 64g + 4i + u for its row i, so the lane reads one float4
        // per 64-channel group.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vr = 16 * kb + 4 * quad + r;
#pragma unroll
                for (int g = 0; g < VG; ++g) {
                    const float4 v = *reinterpret_cast<const float4*>(
                        tile_at<DL>(tile, vr, wv * (Sh::VW / 4) + 16 * g + col));
                    o[4 * g + 0] = mla_mfma(v.x, pr[kb][r], o[4 * g + 0]);
                    o[4 * g + 1] = mla_mfma(v.y, pr[kb][r], o[4 * g + 1]);
                    o[4 * g + 2] = mla_mfma(v.z, pr[kb][r], o[4 * g + 2]);
                    o[4 * g + 3] = mla_mfma(v.w, pr[kb][r], o[4 * g + 3]);
                }
            }
        if (more) stage(buf ^ 1);
    }

    // The row's sum over the four quads' keys; every wave of the group holds
    // the same m, l.
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!live) return;
    const int nsplit = plan.splits;
    const int64_t slot = (int64_t)row * nsplit + sp;
    float* acc = p.part + slot * R + wv * Sh::VW;
    // Lane (col, quad), register rr of block 4g + u: channel 64g + 16*quad + 4*rr + u.
#pragma unroll
    for (int g = 0; g < VG; ++g) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float4 v = make_float4(o[4 * g][rr], o[4 * g + 1][rr], o[4 * g + 2][rr], o[4 * g + 3][rr]);
            *reinterpret_cast<float4*>(acc + 64 * g + 16 * quad + 4 * rr) = v;
        }
    }
    if (wv == 0 && quad == 0) {
        float* ml = p.part + (int64_t)nrows * nsplit * R + slot * 2;
        ml[0] = m;
        ml[1] = l;
    }
}

// Any (R, P): one workgroup per row, every key checked; two passes (the
// row's maximum, then weights and the weighted sum of the latent rows 256
// keys at a time through LDS). Writes the single split's partial state.
__global__ __launch_bounds__(kMlaThreads) void mla_generic_kernel(MlaProblem p) {
    extern __shared__ __align__(16) float lds[];
    const int DL = p.R + p.P;
    float* qrow = lds;                 // DL
    float* acc = qrow + DL;            // R
    float* w = acc + p.R;              // kMlaThreads weights
    float* red = w + kMlaThreads;      // kMlaWaves partials

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int pos = p.vis.pos_offset + row / p.H;
    for (int c = tid; c < DL; c += kMlaThreads) qrow[c] = p.q_abs[(int64_t)row * DL + c];
    for (int c = tid; c < p.R; c += kMlaThreads) acc[c] = 0.0f;
    __syncthreads();

    auto score = [&](int s) {
        const float* srow = p.state + (int64_t)s * DL;
        float d = 0.0f;
        for (int c = 0; c < DL; ++c) d = fmaf(qrow[c], srow[c], d);
        return d * p.qk_scale;
    };
    auto block_reduce = [&](float x, bool is_max) {
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(x, o, 64);
            x = is_max ? fmaxf(x, y) : x + y;
        }
        __syncthreads();
        if ((tid & 63) == 0) red[tid >> 6] = x;
        __syncthreads();
        x = red[0];
        for (int i = 1; i < kMlaWaves; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
        return x;
    };

    float m = -INFINITY;
    for (int s = tid; s < p.S; s += kMlaThreads)
        if (key_visible(p.vis, pos, s)) m = fmaxf(m, score(s));
    m = block_reduce(m, true);

    float l = 0.0f;
    if (m != -INFINITY) {
        for (int s0 = 0; s0 < p.S; s0 += kMlaThreads) {
            const int s = s0 + tid;
            float wt = 0.0f;
            if (s < p.S && key_visible(p.vis, pos, s)) wt = fast_exp2(score(s) - m);
            l += wt;
            __syncthreads();
            w[tid] = wt;
            __syncthreads();
            const int n = p.S - s0 < kMlaThreads ? (int)(p.S - s0) : kMlaThreads;
            for (int c = tid; c < p.R; c += kMlaThreads) {
                float a = acc[c];
                for (int j = 0; j < n; ++j)
                    if (w[j] != 0.0f) a = fmaf(w[j], p.state[(int64_t)(s0 + j) * DL + c], a);
                acc[c] = a;
            }
        }
    }
    l = block_reduce(l, false);
    float* out_acc = p.part + (int64_t)row * p.R;
    for (int c = tid; c < p.R; c += kMlaThreads) out_acc[c] = acc[c];
    if (tid == 0) {
        float* ml = p.part + (int64_t)p.T * p.H * p.R + (int64_t)row * 2;
        ml[0] = m;
        ml[1] = l;
    }
}

// q_abs[t*H + h] = [k_b[h]^T q_nope[t,h] ; q_pe[t,h]], R a multiple of 4.
// grid (H, ceil(R/64), ceil(T/4)), 256 threads: 64 latent channels (16
// float4 columns) of up to 4 query rows. Thread (dg, c4) sums the qk_nope
// rows d = dg, dg + 16, ... of its column with independent 128-bit loads; the
// 16 groups' partial sums are added through LDS in a fixed order.
__global__ __launch_bounds__(kMlaThreads) void mla_absorb4_kernel(MlaProblem p) {
    extern __shared__ __align__(16) float lds[];
    const int N = p.N, R = p.R, P = p.P, DL = R + P;
    float* qn = lds;                                            // [4][N]
    float4* part = reinterpret_cast<float4*>(lds + ((4 * N + 3) & ~3));  // [16][4][16]
    const int tid = threadIdx.x;
    const int c4 = tid & 15, dg = tid >> 4;
    const int h = blockIdx.x;
    const int c = blockIdx.y * 64 + 4 * c4;
    const int t0 = blockIdx.z * 4;
    const int nt = min(4, (int)p.T - t0);
    const int64_t qstride = (int64_t)p.H * (N + P);

    for (int i = tid; i < 4 * N; i += kMlaThreads) {
        const int tr = i / N, d = i % N;
        qn[i] = tr < nt ? p.q[(int64_t)(t0 + tr) * qstride + (int64_t)h * (N + P) + d] : 0.0f;
    }
    __syncthreads();

    float4 a[4];
#pragma unroll
    for (int tr = 0; tr < 4; ++tr) a[tr] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (c < R) {
        const float* kb = p.k_b + (int64_t)h * N * R + c;
        int d = dg;
        for (; d + 48 < N; d += 64) {
            float4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(kb + (int64_t)(d + 16 * u) * R);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) {
                    const float qv = qn[tr * N + d + 16 * u];
                    a[tr].x = fmaf(qv, x[u].x, a[tr].x);
                    a[tr].y = fmaf(qv, x[u].y, a[tr].y);
                    a[tr].z = fmaf(qv, x[u].z, a[tr].z);
                    a[tr].w = fmaf(qv, x[u].w, a[tr].w);
                }
        }
        for (; d < N; d += 16) {
            const float4 x = *reinterpret_cast<const float4*>(kb + (int64_t)d * R);
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
                const float qv = qn[tr * N + d];
                a[tr].x = fmaf(qv, x.x, a[tr].x);
                a[tr].y = fmaf(qv, x.y, a[tr].y);
                a[tr].z = fmaf(qv, x.z, a[tr].z);
                a[tr].w = fmaf(qv, x.w, a[tr].w);
            }
        }
    }
#pragma unroll
    for (int tr = 0; tr < 4; ++tr) part[(dg * 4 + tr) * 16 + c4] = a[tr];
    __syncthreads();
    // Thread (tr, c4) of the first 64 adds the 16 groups for row tr.
    if (tid < 64) {
        const int tr = tid >> 4, cc = tid & 15;
        const int cw = blockIdx.y * 64 + 4 * cc;
        if (tr < nt && cw < R) {
            float4 sum = part[tr * 16 + cc];
            for (int g = 1; g < 16; ++g) {
                const float4 v = part[(g * 4 + tr) * 16 + cc];
                sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
            }
            *reinterpret_cast<float4*>(p.q_abs + ((int64_t)(t0 + tr) * p.H + h) * DL + cw) = sum;
        }
    }
    if (blockIdx.y == 0) {
        const int tr = tid >> 6, lane = tid & 63;
        if (tr < nt) {
            const float* qpe = p.q + (int64_t)(t0 + tr) * qstride + (int64_t)h * (N + P) + N;
            float* dst = p.q_abs + ((int64_t)(t0 + tr) * p.H + h) * DL + R;
            for (int e = lane; e < P; e += 64) dst[e] = qpe[e];
            // The row's slice counter for mla_combine_slice starts at zero.
            if (lane == 0 && p.tickets) p.tickets[(int64_t)(t0 + tr) * p.H + h] = 0u;
        }
    }
}

// q_abs[t*H + h] = [k_b[h]^T q_nope[t,h] ; q_pe[t,h]].
// grid (H, ceil(R/64), ceil(T/4)), 256 threads: 64 latent channels (one per
// lane) of up to 4 query rows; the four waves split the qk_nope contraction
// and add their partial sums through LDS. k_b rows are read coalesced.
__global__ __launch_bounds__(kMlaThreads) void mla_absorb_kernel(MlaProblem p) {
    extern __shared__ __align__(16) float lds[];
    const int N = p.N, R = p.R, P = p.P, DL = R + P;
    float* qn = lds;             // [4][N]: the block's q_nope rows
    float* part = qn + 4 * N;    // [kMlaWaves][4][64]
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int h = blockIdx.x;
    const int c = blockIdx.y * 64 + lane;
    const int t0 = blockIdx.z * 4;
    const int nt = min(4, (int)p.T - t0);
    const int64_t qstride = (int64_t)p.H * (N + P);

    for (int i = tid; i < 4 * N; i += kMlaThreads) {
        const int tr = i / N, d = i % N;
        qn[i] = tr < nt ? p.q[(int64_t)(t0 + tr) * qstride + (int64_t)h * (N + P) + d] : 0.0f;
    }
    __syncthreads();

    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c < R) {
        const float* kb = p.k_b + (int64_t)h * N * R + c;
        for (int d = wave; d < N; d += kMlaWaves) {
            const float x = kb[(int64_t)d * R];
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) a[tr] = fmaf(qn[tr * N + d], x, a[tr]);
        }
    }
#pragma unroll
    for (int tr = 0; tr < 4; ++tr) part[(wave * 4 + tr) * 64 + lane] = a[tr];
    __syncthreads();
    // Wave tr writes row tr (fixed summation order over the waves).
    if (wave < nt && c < R) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kMlaWaves; ++w) sum += part[(w * 4 + wave) * 64 + lane];
        p.q_abs[((int64_t)(t0 + wave) * p.H + h) * DL + c] = sum;
    }
    if (blockIdx.y == 0 && wave < nt) {
        const float* qpe = p.q + (int64_t)(t0 + wave) * qstride + (int64_t)h * (N + P) + N;
        float* dst = p.q_abs + ((int64_t)(t0 + wave) * p.H + h) * DL + R;
        for (int e = lane; e < P; e += 64) dst[e] = qpe[e];
        if (lane == 0 && p.tickets) p.tickets[(int64_t)(t0 + wave) * p.H + h] = 0u;
    }
}

// out[t, h*Dv + e] = v_b[h][e] . o_lat, o_lat the merge of the splits'
// partial states: M = max m_i, L = sum l_i 2^(m_i - M),
// o_lat = sum acc_i 2^(m_i - M) / L. A row with no visible key outputs 0.
// grid (T*H, ceil(Dv/32)), 256 threads; each wave takes 8 output channels.
__global__ __launch_bounds__(kMlaThreads) void mla_combine_kernel(MlaProblem p, int nsplit) {
    extern __shared__ __align__(16) float lds[];
    float* olat = lds;               // R
    float* wts = olat + p.R;         // nsplit
    float* red = wts + nsplit;       // kMlaWaves
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int row = blockIdx.x;
    const int h = row % p.H;
    const int e0 = blockIdx.y * 32;
    const int R = p.R;
    const float* ml = p.part + (int64_t)p.T * p.H * nsplit * R + (int64_t)row * nsplit * 2;
    const float* acc = p.part + (int64_t)row * nsplit * R;
    float* orow = p.out + (int64_t)row * p.Dv;

    auto block_reduce = [&](float x, bool is_max) {
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(x, o, 64);
            x = is_max ? fmaxf(x, y) : x + y;
        }
        __syncthreads();
        if (lane == 0) red[wave] = x;
        __syncthreads();
        x = red[0];
        for (int i = 1; i < kMlaWaves; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
        return x;
    };

    float mx = -INFINITY;
    for (int i = tid; i < nsplit; i += kMlaThreads) mx = fmaxf(mx, ml[2 * i]);
    const float M = block_reduce(mx, true);
    if (M == -INFINITY) {  // no visible key in any split
        if (tid < 32 && e0 + tid < p.Dv) orow[e0 + tid] = 0.0f;
        return;
    }
    float ls = 0.0f;
    for (int i = tid; i < nsplit; i += kMlaThreads) {
        const float wi = fast_exp2(ml[2 * i] - M);
        wts[i] = wi;
        ls += ml[2 * i + 1] * wi;
    }
    const float L = block_reduce(ls, false);  // its barriers also publish wts
    const float inv = 1.0f / L;
    for (int c = tid; c < R; c += kMlaThreads) {
        float a = 0.0f;
        for (int i = 0; i < nsplit; ++i) a = fmaf(acc[(int64_t)i * R + c], wts[i], a);
        olat[c] = a * inv;
    }
    __syncthreads();

    for (int k = 0; k < 8; ++k) {
        const int e = e0 + wave * 8 + k;
        if (e >= p.Dv) break;  // wave-uniform
        const float* vb = p.v_b + ((int64_t)h * p.Dv + e) * R;
        float d = 0.0f;
        for (int c = lane; c < R; c += 64) d = fmaf(vb[c], olat[c], d);
        for (int o = 32; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
        if (lane == 0) orow[e] = d;
    }
}

// The same merge and projection for R a multiple of 4 (R/4 <= 256 float4
// columns), laid out for few rows: 1024 threads per workgroup, and every
// thread first requests its splits' (max, sum) pairs, its first kBatch
// accumulator float4s and the v_b rows it will project, so one memory round
// trip covers nearly all of them. grid (T*H, ceil(Dv/32)). The splits'
// accumulators are summed by G = 1024 / (R/4) thread groups (split i to
// group i % G), then added through LDS in a fixed order; each of the 16
// waves projects 2 output channels.
constexpr int kCombThreads = 1024;
constexpr int kCombWaves = kCombThreads / 64;
constexpr int kCombBatch = 8;    // accumulator float4s requested up front per thread

// OUT: output channels per workgroup (32: 2 per wave; 16: 1 per wave).
template <int OUT>
__global__ __launch_bounds__(kCombThreads) void mla_combine4_kernel(MlaProblem p, int nsplit) {
    constexpr int EPW = OUT / kCombWaves;
    extern __shared__ __align__(16) float lds[];
    const int R = p.R, C4 = R / 4;
    float4* olat4 = reinterpret_cast<float4*>(lds);             // C4
    float4* gpart = olat4 + C4;                                   // [G][C4]
    float* wts = reinterpret_cast<float*>(gpart + kCombThreads);  // nsplit
    float* red = wts + nsplit;                                    // kCombWaves
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int row = blockIdx.x;
    const int h = row % p.H;
    const int e0 = blockIdx.y * OUT;
    const float* ml = p.part + (int64_t)p.T * p.H * nsplit * R + (int64_t)row * nsplit * 2;
    const float4* acc4 = reinterpret_cast<const float4*>(p.part + (int64_t)row * nsplit * R);
    float* orow = p.out + (int64_t)row * p.Dv;
    const int G = kCombThreads / C4;
    const int gi = tid / C4, c4 = tid % C4;
    const bool summer = gi < G;

    // Requests first: (max, sum) pairs, accumulators, v_b rows.
    const float2 mlv = tid < nsplit ? *reinterpret_cast<const float2*>(ml + 2 * tid) : make_float2(-INFINITY, 0.0f);
    float4 xa[kCombBatch];
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
        const int i = gi + u * G;
        xa[u] = summer && i < nsplit ? acc4[(int64_t)i * C4 + c4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    constexpr int kVj = 256 / 64;  // float4s of a v_b row per lane (R/4 <= 256)
    float4 vb[EPW][kVj];
#pragma unroll
    for (int k = 0; k < EPW; ++k) {
        const int e = e0 + EPW * wave + k;
#pragma unroll
        for (int j = 0; j < kVj; ++j) {
            const int c = lane + 64 * j;
            vb[k][j] = e < p.Dv && c < C4
                           ? *reinterpret_cast<const float4*>(p.v_b + ((int64_t)h * p.Dv + e) * R + 4 * c)
                           : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

    auto block_reduce = [&](float x, bool is_max) {
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(x, o, 64);
            x = is_max ? fmaxf(x, y) : x + y;
        }
        __syncthreads();
        if (lane == 0) red[wave] = x;
        __syncthreads();
        x = red[0];
        for (int i = 1; i < kCombWaves; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
        return x;
    };

    // nsplit <= 1024: one pair per thread.
    const float M = block_reduce(mlv.x, true);
    if (M == -INFINITY) {  // no visible key in any split
        if (tid < OUT && e0 + tid < p.Dv) orow[e0 + tid] = 0.0f;
        return;
    }
    float ls = 0.0f;
    if (tid < nsplit) {
        const float wi = fast_exp2(mlv.x - M);
        wts[tid] = wi;
        ls = mlv.y * wi;
    }
    const float L = block_reduce(ls, false);  // its barriers also publish wts
    const float inv = 1.0f / L;

    if (summer) {
        float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const int i = gi + u * G;
            const float wv = i < nsplit ? wts[i] : 0.0f;
            a.x = fmaf(xa[u].x, wv, a.x);
            a.y = fmaf(xa[u].y, wv, a.y);
            a.z = fmaf(xa[u].z, wv, a.z);
            a.w = fmaf(xa[u].w, wv, a.w);
        }
        // Further splits, kCombBatch at a time.
        for (int i0 = gi + kCombBatch * G; i0 < nsplit; i0 += kCombBatch * G) {
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) {
                const int i = i0 + u * G;
                xa[u] = i < nsplit ? acc4[(int64_t)i * C4 + c4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) {
                const int i = i0 + u * G;
                const float wv = i < nsplit ? wts[i] : 0.0f;
                a.x = fmaf(xa[u].x, wv, a.x);
                a.y = fmaf(xa[u].y, wv, a.y);
                a.z = fmaf(xa[u].z, wv, a.z);
                a.w = fmaf(xa[u].w, wv, a.w);
            }
        }
        gpart[gi * C4 + c4] = a;
    }
    __syncthreads();
    for (int c = tid; c < C4; c += kCombThreads) {
        float4 sum = gpart[c];
        for (int g = 1; g < G; ++g) {
            const float4 v = gpart[g * C4 + c];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        olat4[c] = make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    }
    __syncthreads();

    // Wave w projects channels e0 + 2w and e0 + 2w + 1: lanes stride the
    // latent channels in float4s, then the wave adds them up.
    float d[EPW];
#pragma unroll
    for (int k = 0; k < EPW; ++k) d[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < kVj; ++j) {
        const int c = lane + 64 * j;
        if (c < C4) {
            const float4 o = olat4[c];
#pragma unroll
            for (int k = 0; k < EPW; ++k)
                d[k] = fmaf(vb[k][j].x, o.x, fmaf(vb[k][j].y, o.y, fmaf(vb[k][j].z, o.z, fmaf(vb[k][j].w, o.w, d[k]))));
        }
    }
#pragma unroll
    for (int k = 0; k < EPW; ++k) {
        float x = d[k];
        for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
        const int e = e0 + EPW * wave + k;
        if (lane == 0 && e < p.Dv) orow[e] = x;
    }
}

// The merge split by latent channels instead of outputs: grid (T*H, R/64),
// 256 threads. Workgroup (row, slice) merges the row's splits over its 64
// latent channels only (so every partial accumulator is read once per call)
// and multiplies them by the matching 64 columns of v_b[h], which gives the
// slice's share of all Dv outputs:
//   y[slice][e] = sum over c in the slice of v_b[h][e][c] o_lat[c].
// out[e] is the sum of the slices' shares, added in slice order by whichever
// workgroup of the row finishes last (a counter per row, zeroed by
// mla_absorb earlier in the call). The shares are agent-scope atomic stores,
// which reach the memory every XCD sees before the store completes; each
// wave waits for its stores to complete before the workgroup takes its
// ticket, and the last workgroup reads the shares with agent-scope atomic
// loads, which do not hit a stale cached copy. (An agent-scope release fence
// would write back the whole L2 of the XCD for each workgroup, which costs far
// more than these few hundred bytes.)
constexpr int kSliceW = 64;                   // latent channels per slice
constexpr int kSliceC4 = kSliceW / 4;         // their float4 columns
constexpr int kSliceGroups = kMlaThreads / kSliceC4;  // split groups (16)
constexpr int kSliceBatch = 8;                // accumulator float4s requested up front per thread
constexpr int kSliceMaxDv = 256;
constexpr int kSliceMax = 8;                 // slices per row (R <= 512)

__global__ __launch_bounds__(kMlaThreads) void mla_combine_slice_kernel(MlaProblem p, int nsplit) {
    __shared__ float4 s_part[kSliceGroups][kSliceC4];
    __shared__ float4 s_olat[kSliceC4];
    __shared__ float s_w[kMlaMaxSplits];
    __shared__ float s_red[kMlaWaves];
    __shared__ uint32_t s_ticket;
    const int R = p.R, C4 = R / 4;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int row = blockIdx.x;
    const int slice = blockIdx.y, nslices = gridDim.y;
    const int h = row % p.H;
    const int sg = tid / kSliceC4, c4 = tid % kSliceC4;
    const float* ml = p.part + (int64_t)p.T * p.H * nsplit * R + (int64_t)row * nsplit * 2;
    const float4* acc4 = reinterpret_cast<const float4*>(p.part + (int64_t)row * nsplit * R) + slice * kSliceC4 + c4;

    // Requests first: (max, sum) pairs, accumulator columns, v_b columns.
    constexpr int kPairs = kMlaMaxSplits / kMlaThreads;
    float2 mlv[kPairs];
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const int i = tid + j * kMlaThreads;
        mlv[j] = i < nsplit ? *reinterpret_cast<const float2*>(ml + 2 * i) : make_float2(-INFINITY, 0.0f);
    }
    float4 xa[kSliceBatch];
#pragma unroll
    for (int u = 0; u < kSliceBatch; ++u) {
        const int i = sg + u * kSliceGroups;
        xa[u] = i < nsplit ? acc4[(int64_t)i * C4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    // Output e = 64 k + tid / 4 takes slice channels 16 q .. 16 q + 15 (q = tid % 4).
    constexpr int kPass = kSliceMaxDv / 64;
    const int eq = tid >> 2, q = tid & 3;
    float4 vb[kPass][4];
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
        const int e = 64 * k + eq;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            vb[k][j] = e < p.Dv ? *reinterpret_cast<const float4*>(p.v_b + ((int64_t)h * p.Dv + e) * R +
                                                                    slice * kSliceW + 16 * q + 4 * j)
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }

    auto block_reduce = [&](float x, bool is_max) {
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(x, o, 64);
            x = is_max ? fmaxf(x, y) : x + y;
        }
        __syncthreads();
        if (lane == 0) s_red[wave] = x;
        __syncthreads();
        x = s_red[0];
        for (int i = 1; i < kMlaWaves; ++i) x = is_max ? fmaxf(x, s_red[i]) : x + s_red[i];
        return x;
    };

    float mx = mlv[0].x;
#pragma unroll
    for (int j = 1; j < kPairs; ++j) mx = fmaxf(mx, mlv[j].x);
    const float M = block_reduce(mx, true);
    // No visible key in any split: every weight is zero and so is the row.
    float ls = 0.0f;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const int i = tid + j * kMlaThreads;
        if (i < nsplit) {
            const float wi = M == -INFINITY ? 0.0f : fast_exp2(mlv[j].x - M);
            s_w[i] = wi;
            ls = fmaf(mlv[j].y, wi, ls);
        }
    }
    const float L = block_reduce(ls, false);  // its barriers also publish s_w
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;

    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int i0 = sg;; i0 += kSliceBatch * kSliceGroups) {
#pragma unroll
        for (int u = 0; u < kSliceBatch; ++u) {
            const int i = i0 + u * kSliceGroups;
            const float wv = i < nsplit ? s_w[i] : 0.0f;
            a.x = fmaf(xa[u].x, wv, a.x);
            a.y = fmaf(xa[u].y, wv, a.y);
            a.z = fmaf(xa[u].z, wv, a.z);
            a.w = fmaf(xa[u].w, wv, a.w);
        }
        const int next = i0 + kSliceBatch * kSliceGroups;
        if (next >= nsplit) break;
#pragma unroll
        for (int u = 0; u < kSliceBatch; ++u) {
            const int i = next + u * kSliceGroups;
            xa[u] = i < nsplit ? acc4[(int64_t)i * C4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
    s_part[sg][c4] = a;
    __syncthreads();
    if (tid < kSliceC4) {
        float4 sum = s_part[0][tid];
        for (int g = 1; g < kSliceGroups; ++g) {
            const float4 v = s_part[g][tid];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        s_olat[tid] = make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    }
    __syncthreads();

    // This slice's share of every output: four lanes per output, then their sum.
    float* ys = p.yslice + ((int64_t)row * nslices + slice) * p.Dv;
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
        const int e = 64 * k + eq;
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 o = s_olat[4 * q + j];
            d = fmaf(vb[k][j].x, o.x, fmaf(vb[k][j].y, o.y, fmaf(vb[k][j].z, o.z, fmaf(vb[k][j].w, o.w, d))));
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        if (q == 0 && e < p.Dv) __hip_atomic_store(ys + e, d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Every wave's shares have completed before the ticket is taken.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(p.tickets + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != (uint32_t)(nslices - 1)) return;
    const float* yr = p.yslice + (int64_t)row * nslices * p.Dv;
    float* orow = p.out + (int64_t)row * p.Dv;
    for (int e = tid; e < p.Dv; e += kMlaThreads) {
        // All the row's shares requested before any is added.
        float y[kSliceMax];
#pragma unroll
        for (int sl = 0; sl < kSliceMax; ++sl)
            y[sl] = sl < nslices ? __hip_atomic_load(yr + (int64_t)sl * p.Dv + e, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0.0f;
        float sum = y[0];
#pragma unroll
        for (int sl = 1; sl < kSliceMax; ++sl)
            if (sl < nslices) sum += y[sl];
        orow[e] = sum;
    }
}

template <int R, int P>
hipError_t launch_split_rp(const MlaProblem& p, const MlaPlan& plan, const Launch& L) {
    if (plan.row_groups == 2) {
        const dim3 grid((unsigned)plan.splits, (unsigned)((plan.row_blocks + 1) / 2));
        return launch_kernel(mla_split_kernel<R, P, 2>, grid, dim3(kMlaThreads * 2),
                             (uint32_t)MlaShape<R, P, 2>::lds_bytes, L, p, plan);
    }
    if (plan.row_groups != 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)plan.splits, (unsigned)plan.row_blocks);
    return launch_kernel(mla_split_kernel<R, P, 1>, grid, dim3(kMlaThreads), (uint32_t)MlaShape<R, P, 1>::lds_bytes,
                         L, p, plan);
}

}  // namespace

bool mla_fast_supported(int R, int P) { return (R == 512 || R == 256) && P == 64; }
bool mla_slices_supported(int R, int Dv) {
    return R % kSliceW == 0 && R / kSliceW <= kSliceMax && Dv >= 1 && Dv <= kSliceMaxDv;
}

hipError_t launch_mla_absorb(const MlaProblem& p, const Launch& L) {
    const dim3 grid((unsigned)p.H, (unsigned)((p.R + 63) / 64), (unsigned)((p.T + 3) / 4));
    if (p.R % 4 == 0) {
        const size_t lds = sizeof(float) * (size_t)((4 * p.N + 3) & ~3) + sizeof(float4) * 16 * 4 * 16;
        return launch_kernel(mla_absorb4_kernel, grid, dim3(kMlaThreads), (uint32_t)lds, L, p);
    }
    const size_t lds = sizeof(float) * (4 * (size_t)p.N + kMlaWaves * 4 * 64);
    return launch_kernel(mla_absorb_kernel, grid, dim3(kMlaThreads), (uint32_t)lds, L, p);
}

hipError_t launch_mla_split(const MlaProblem& p, const MlaPlan& plan, const Launch& L) {
    if (plan.splits < 1 || plan.splits > kMlaMaxSplits) return hipErrorInvalidValue;
    if (plan.fast) {
        if (p.R == 512 && p.P == 64) return launch_split_rp<512, 64>(p, plan, L);
        if (p.R == 256 && p.P == 64) return launch_split_rp<256, 64>(p, plan, L);
        return hipErrorInvalidValue;
    }
    if (plan.splits != 1) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * ((size_t)p.R + p.P + p.R + kMlaThreads + kMlaWaves);
    return launch_kernel(mla_generic_kernel, dim3((unsigned)(p.T * p.H)), dim3(kMlaThreads), (uint32_t)lds,
                         L, p);
}

hipError_t launch_mla_combine(const MlaProblem& p, const MlaPlan& plan, const Launch& L) {
    if (plan.splits < 1 || plan.splits > kMlaMaxSplits) return hipErrorInvalidValue;
    if (plan.slices > 0) {
        if (!mla_slices_supported(p.R, p.Dv) || plan.slices != p.R / kSliceW || !p.yslice || !p.tickets)
            return hipErrorInvalidValue;
        const dim3 grid((unsigned)(p.T * p.H), (unsigned)plan.slices);
        return launch_kernel(mla_combine_slice_kernel, grid, dim3(kMlaThreads), 0, L, p, plan.splits);
    }
    if (p.R % 4 == 0 && p.R / 4 <= 256) {
        const size_t lds = sizeof(float4) * ((size_t)p.R / 4 + kCombThreads) + sizeof(float) * (plan.splits + kCombWaves);
        if (plan.combine_out == 16) {
            const dim3 grid((unsigned)(p.T * p.H), (unsigned)((p.Dv + 15) / 16));
            return launch_kernel(mla_combine4_kernel<16>, grid, dim3(kCombThreads), (uint32_t)lds, L, p, plan.splits);
        }
        const dim3 grid((unsigned)(p.T * p.H), (unsigned)((p.Dv + 31) / 32));
        return launch_kernel(mla_combine4_kernel<32>, grid, dim3(kCombThreads), (uint32_t)lds, L, p, plan.splits);
    }
    const dim3 grid((unsigned)(p.T * p.H), (unsigned)((p.Dv + 31) / 32));
    const size_t lds = sizeof(float) * ((size_t)p.R + plan.splits + kMlaWaves);
    return launch_kernel(mla_combine_kernel, grid, dim3(kMlaThreads), (uint32_t)lds, L, p, plan.splits);
}

}  // namespace attn
