// Decode path of op `attention` on the matrix cores, for groups of many query
// rows per KV head (graph protocol op catalogue, op `attention`: several query
// heads share a key/value head, param kvHeads; a few query rows against a
// long cached key range). Like decode_split it reads every visible K and V
// row of a KV head once, for all the query rows of that head's group, and
// leaves per-split partial states for decode_combine; it differs in where the
// arithmetic runs: the score and weighted-sum contractions go to
// v_mfma_f32_16x16x4f32, so the vector ALUs only run the softmax, and the
// work per key no longer grows with the number of rows in the group.
//
// decode_mfma: grid (splits, kv_heads), 256 threads (1-D on appending calls,
// as decode_split). The workgroup's four waves take the split's key rows in
// tiles of 16 (wave w: tiles w, w + 4, ...), each with its own online
// softmax over the group's rows (up to 16 per row block, NB blocks), and
// merge through LDS at the end. A tile's K and V rows are loaded row by row
// (each load instruction of a wave reads whole row slices), pass through the
// wave's own LDS area and come out laid out as the MFMA wants them (lane l,
// column n = l % 16, lane group kg = l / 16):
//   scores S^T = K Q^T, one MFMA per 4 channels: A[key i][k] in lane i + 16k
//     holds K[key][d], B[k][query j] in lane j + 16k holds q[query][d], for
//     the channel d = 16 m + 4 kg + c of step (m, c): lane l takes 16 bytes
//     of K row n at 64-byte steps. The result D[key i][query j] sits
//     in lane j + 16 (i / 4), element i % 4: lane l holds the scores of
//     keys 4 kg .. 4 kg + 3 for query n.
//   weighted sum O^T += V^T P^T, step r contracting keys 4k + r: A[e][k] =
//     V[key 4 kg + r][e] with e = 64 h + 4 n + c for output block (h, c),
//     B[k][query j] = the weight in element r of lane j + 16 k, which is
//     exactly where the scores left it. The accumulator of block (h, c)
//     holds, in lane l element i, O[query n][e = 64 h + 16 kg + 4 i + c]:
//     for each h a lane holds 16 consecutive outputs of one query.
// Running maxima are kept per query and shared by its four lane groups (two
// lane shuffles per tile), with the same lazy reference (weights up to 2^8)
// and base-2 domain as decode_split.
#include "device_common.h"
#include "rope_device.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;      // keys per wave tile: the MFMA's M
constexpr float kLazy = 8.0f;  // log2 of the largest weight before the reference max moves
constexpr int kMaxSplits = 1024;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Component c of a float4 (c is a constant once the loops are unrolled).
__device__ __forceinline__ float comp(const float4& v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// Orders one wave's LDS writes and its lanes' later reads of them (and
// reads before later writes): a wave's LDS instructions complete in order,
// so only the compiler must not move accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// D: key/query width, DV: value width, NB: blocks of 16 query rows per KV
// group, EPI: softcap / ALiBi / bias possible (else the score is the scaled
// product and q carries the scale).
// Built for one workgroup per CU where headDim + vHeadDim >= 256 (the
// planner's choice there; the raw rows, the matrix-layout copies and the
// accumulators then have a SIMD's 512 registers), else two.
template <int D, int DV, int NB, bool EPI>
__global__ __launch_bounds__(kThreads, (D + DV >= 256 ? 1 : 2)) void decode_mfma_kernel(Problem p, DecodePlan plan,
                                                                                       float* __restrict__ ws) {
    constexpr int KM = D / 16;   // float4 of a K row per lane (4 channels each of KM 16-channel steps)
    constexpr int VH = DV / 64;  // float4 of each of 4 V rows per lane
    constexpr int NO = 4 * VH;   // output blocks of 16 values per row block
    constexpr int KT4 = D / 4, VT4 = DV / 4;  // float4s per K / V row
    constexpr int KR = kTile * KT4 / 64, VR = kTile * VT4 / 64;  // raw float4 loads per lane per tile
    static_assert(kTile * KT4 % 64 == 0 && kTile * VT4 % 64 == 0, "a tile's rows must split evenly over a wave");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kg = lane >> 4;
    // LDS: each wave's K area [kTile][KT4] and V area [kTile][VT4] float4s
    // (float4 c of row r at c ^ (r & 15): both the row-wise writes and the
    // matrix-layout reads hit distinct bank groups), then the merge's
    // (max, sum) pairs.
    extern __shared__ float4 lds4[];
    float4* wk = lds4 + wave * kTile * KT4;
    float4* wv = lds4 + kWaves * kTile * KT4 + wave * kTile * VT4;

    // Split sp of KV group g (appending calls: the append splits last).
    int sp, g;
    if (plan.k_new) {
        const int per = plan.splits - 1;
        const int near_sp = plan.splits - 1 - (plan.sink_hi > 0 ? 1 : 0);
        const int id = blockIdx.x;
        if (id < per * p.G) {
            g = id / per;
            const int x = id - g * per;
            sp = x < near_sp ? x : x + 1;
        } else {
            g = id - per * p.G;
            sp = near_sp;
        }
    } else {
        sp = blockIdx.x;
        g = blockIdx.y;
    }
    const int hpg = p.H / p.G;
    const int nrows = (int)p.T * hpg;

    // This lane's query rows: column n of each row block (row 16 b + n is
    // query row t = r / hpg of head g * hpg + r % hpg; rows past nrows are
    // padding, computed on zeros and never written).
    int tt[NB], hh[NB], pos[NB];
    bool live[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int r = 16 * b + n;
        live[b] = r < nrows;
        tt[b] = live[b] ? r / hpg : 0;
        hh[b] = g * hpg + (live[b] ? r % hpg : 0);
        pos[b] = p.ep.pos_offset + tt[b];
    }
    float slope[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) slope[b] = alibi_slope(p.ep, hh[b]);

    // The split's keys, walked in tiles of 16 rows (decode_split's walk, in
    // tile units): a chunk (possibly from a rotated start), interleaved
    // blocks, the sink keys, or the near / appended rows.
    const bool sink_split = plan.sink_hi > 0 && sp == plan.splits - 1;
    const bool near_split = plan.near_hi > plan.near_lo && sp == plan.splits - 1 - (plan.sink_hi > 0 ? 1 : 0);
    const bool append = near_split && plan.k_new != nullptr;
    const bool spread = plan.block > 0 && !sink_split && !near_split;
    int k0, k1, nw, bsh, bstride = 1, boff = 0, bwrap = INT_MAX;
    if (spread) {
        k0 = (int)plan.range.lo;
        k1 = (int)plan.range.hi;
        bsh = 31 - __builtin_clz((unsigned)plan.block);
        const int nblocks = (k1 - k0 + plan.block - 1) >> bsh;
        nw = ((nblocks - 1 - sp) / plan.main_splits + 1) << bsh;
        bstride = plan.main_splits;
        boff = sp;
    } else {
        k0 = sink_split ? 0 : near_split ? plan.near_lo : (int)(plan.range.lo + (int64_t)sp * plan.chunk);
        k1 = sink_split   ? plan.sink_hi
             : near_split ? plan.near_hi
                          : (int)min(plan.range.hi, (int64_t)k0 + plan.chunk);
        nw = k1 - k0;
        bsh = 4;  // tiles of 16 rows
        if (plan.rotate > 0 && nw > 0 && nw % kTile == 0) {
            boff = (int)(((int64_t)sp * plan.rotate) % nw) >> bsh;
            bwrap = nw >> bsh;
        }
    }
    auto tile_row = [&](int j) {
        const int w = j * kTile;
        int b = (w >> bsh) * bstride + boff;
        if (b >= bwrap) b -= bwrap;
        return k0 + (b << bsh) + (w & ((1 << bsh) - 1));
    };
    const int ntiles = (nw + kTile - 1) / kTile;
    const bool dense = chunk_all_visible(p.ep, p.ep.pos_offset, p.ep.pos_offset + (int)p.T - 1, k0, k1);

    // Workgroup-uniform bases, 32-bit per-lane offsets (the host keeps a
    // split's rows times the row stride below 2^31 floats).
    const uint32_t kstride = (uint32_t)(p.G * D), vstride = (uint32_t)(p.G * DV);
    const float* kwg = (append ? plan.k_new : p.k + (int64_t)k0 * kstride) + (int64_t)g * D;
    const float* vwg = (append ? plan.v_new : p.v + (int64_t)k0 * vstride) + (int64_t)g * DV;

    // A tile's K and V rows come from memory row by row (each load
    // instruction of a wave reads whole row slices: 2 rows of 512 bytes at
    // headDim 128), into the wave's own LDS area, and from there into the
    // matrix layouts above. (Loaded straight in the matrix layout, each K
    // instruction touched 64 bytes of 16 different rows: a load-only kernel
    // with that pattern streamed 64/8-head-shaped K/V at 6.0 TB/s, with
    // whole-row loads and the trip through LDS at 6.5 TB/s.) A tile's K goes
    // out once the previous tile's K has moved to LDS, its V once the
    // previous V has, and its bias entries once the previous weighted sum is
    // done. The first tile's loads go out before q is fetched. Rows past the
    // split's end read its last row and are masked.
    float4 kr[KR], vr[VR];
    float bf[NB][4];
    auto load_k = [&](int j) {
        const int s0 = tile_row(j);
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int f = 64 * i + lane, row = f / KT4, c4 = f - row * KT4;
            const uint32_t rk = (uint32_t)(min(s0 + row, k1 - 1) - k0);
            kr[i] = load_stream4(kwg + rk * kstride + 4 * c4);
        }
    };
    auto load_v = [&](int j) {
        const int s0 = tile_row(j);
#pragma unroll
        for (int i = 0; i < VR; ++i) {
            const int f = 64 * i + lane, row = f / VT4, c4 = f - row * VT4;
            const uint32_t rv = (uint32_t)(min(s0 + row, k1 - 1) - k0);
            vr[i] = load_stream4(vwg + rv * vstride + 4 * c4);
        }
    };
    auto load_bias = [&](int j) {
        const int s0 = tile_row(j);
        if constexpr (EPI) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int sc = min(s0 + 4 * kg + r, k1 - 1);
                    float x = 0.0f;
                    if (p.ep.bias_kind == ATTN_BIAS_TS) x = p.bias[(int64_t)tt[b] * p.S + sc];
                    else if (p.ep.bias_kind == ATTN_BIAS_HTS) x = p.bias[((int64_t)hh[b] * p.T + tt[b]) * p.S + sc];
                    bf[b][r] = x;
                }
        }
    };
    if (wave < ntiles) {
        load_k(wave);
        load_v(wave);
        load_bias(wave);
    }

    // q, in the B layout: lane l holds channels 16 m + 4 kg .. + 3 of its
    // row's query, turned by the rotary embedding when there is one.
    float4 qf[NB][KM];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float* head = p.q + (int64_t)tt[b] * p.H * D + (int64_t)hh[b] * D;
#pragma unroll
        for (int m = 0; m < KM; ++m) {
            float4 x = zero4();
            if (live[b]) {
                x = p.rope.on ? rope_channels4(p.rope, head, 16 * m + 4 * kg, p.rope.pos0 + tt[b])
                              : *reinterpret_cast<const float4*>(head + 16 * m + 4 * kg);
            }
            if constexpr (!EPI) {
                const float c = p.ep.scale * kLog2e;
                x.x *= c; x.y *= c; x.z *= c; x.w *= c;
            }
            qf[b][m] = x;
        }
    }

    f32x4v acc[NB][NO];
    float mrow[NB], lsum[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        mrow[b] = -INFINITY;
        lsum[b] = 0.0f;
#pragma unroll
        for (int o = 0; o < NO; ++o) acc[b][o] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    }

    for (int j = wave; j < ntiles; j += kWaves) {
        const int s0 = tile_row(j);
        const bool more = j + kWaves < ntiles;
        // K: raw rows into LDS, back out in the A layout (row n, channels
        // 16 m + 4 kg .. + 3); then the next tile's K goes out.
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int f = 64 * i + lane, row = f / KT4, c4 = f - row * KT4;
            wk[row * KT4 + (c4 ^ (row & 15))] = kr[i];
        }
        wave_lds_sync();
        float4 kf[KM];
#pragma unroll
        for (int m = 0; m < KM; ++m) kf[m] = wk[n * KT4 + ((4 * m + kg) ^ n)];
        // Appended rows go on into the caches: each lane stores the row
        // slices it loaded (every element of the tile exactly once).
        if (append) {
            float* kd = plan.k_cache + (int64_t)k0 * kstride + (int64_t)g * D;
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                const int f = 64 * i + lane, row = f / KT4, c4 = f - row * KT4;
                if (s0 + row < k1)
                    *reinterpret_cast<float4*>(kd + ((uint32_t)(s0 + row - k0) * kstride + 4 * c4)) = kr[i];
            }
        }
        if (more) load_k(j + kWaves);
        // Scores of keys s0 + 4 kg + i for this lane's query of each block.
        f32x4v sc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4v s = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < KM; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) s = mfma16(comp(kf[m], c), comp(qf[b][m], c), s);
            sc[b] = s;
        }
        __builtin_amdgcn_sched_barrier(0);  // V's trip through LDS after the score work
        // V: raw rows into LDS, back out in the A layout of the weighted sum
        // (rows 4 kg + r, channels 64 h + 4 n .. + 3); then the next V.
#pragma unroll
        for (int i = 0; i < VR; ++i) {
            const int f = 64 * i + lane, row = f / VT4, c4 = f - row * VT4;
            wv[row * VT4 + (c4 ^ (row & 15))] = vr[i];
        }
        wave_lds_sync();
        float4 vf[4][VH];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int h = 0; h < VH; ++h) vf[r][h] = wv[(4 * kg + r) * VT4 + ((16 * h + n) ^ ((4 * kg + r) & 15))];
        if (append) {
            float* vd = plan.v_cache + (int64_t)k0 * vstride + (int64_t)g * DV;
#pragma unroll
            for (int i = 0; i < VR; ++i) {
                const int f = 64 * i + lane, row = f / VT4, c4 = f - row * VT4;
                if (s0 + row < k1)
                    *reinterpret_cast<float4*>(vd + ((uint32_t)(s0 + row - k0) * vstride + 4 * c4)) = vr[i];
            }
        }
        if (more) load_v(j + kWaves);

        const bool check = !(dense && s0 + kTile <= k1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = s0 + 4 * kg + i;
                float v = sc[b][i];
                if constexpr (EPI) v = score_epilogue(v, p.ep, slope[b], pos[b], s, bf[b][i]) * kLog2e;
                if (check) {
                    const bool vis = live[b] & (s < k1) & key_visible(p.ep, pos[b], s);
                    if (!vis) v = -INFINITY;
                }
                x[i] = v;
            }
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            if (mx > mrow[b] + kLazy) {
                const float alpha = fast_exp2(mrow[b] - mx);
                lsum[b] *= alpha;
#pragma unroll
                for (int o = 0; o < NO; ++o) acc[b][o] *= alpha;
                mrow[b] = mx;
            }
            const float mu = mrow[b] == -INFINITY ? 0.0f : mrow[b];
            float pw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[i] = fast_exp2(x[i] - mu);
                lsum[b] += pw[i];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int h = 0; h < VH; ++h)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[b][4 * h + c] = mfma16(comp(vf[r][h], c), pw[r], acc[b][4 * h + c]);
        }
        if (more) load_bias(j + kWaves);
        wave_lds_sync();  // this tile's LDS reads come before the next tile's writes
    }

    // Each query's sum over its four lane groups, then the four waves merge
    // through LDS, one row block at a time; a wave's share of the merge goes
    // into its own V area ([16][DV / 4] float4s).
    float* s_m = reinterpret_cast<float*>(lds4 + kWaves * kTile * (KT4 + VT4));  // [kWaves][16]
    float* s_l = s_m + kWaves * 16;                                               // [kWaves][16]
    auto s_acc = [&](int w, int rn, int e4) -> float4& { return lds4[kWaves * kTile * KT4 + w * kTile * VT4 + rn * VT4 + e4]; };
    const int nsplit = plan.splits;
    float* ws_acc = ws;
    float* ws_ml = ws + (int64_t)p.T * p.H * nsplit * DV;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float l = lsum[b];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (b > 0) __syncthreads();  // the previous block's merge has read s_*
        if (kg == 0) {
            s_m[wave * 16 + n] = mrow[b];
            s_l[wave * 16 + n] = l;
        }
#pragma unroll
        for (int h = 0; h < VH; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_acc(wave, n, 16 * h + 4 * kg + i) =
                    make_float4(acc[b][4 * h][i], acc[b][4 * h + 1][i], acc[b][4 * h + 2][i], acc[b][4 * h + 3][i]);
        __syncthreads();
        for (int idx = tid; idx < 16 * (DV / 4); idx += kThreads) {
            const int rn = idx / (DV / 4), e4 = idx % (DV / 4);
            const int r = 16 * b + rn;
            if (r >= nrows) continue;
            float M = s_m[rn];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w * 16 + rn]);
            const float Mu = M == -INFINITY ? 0.0f : M;
            float L = 0.0f;
            float4 A = zero4();
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = fast_exp2(s_m[w * 16 + rn] - Mu);
                L += s_l[w * 16 + rn] * f;
                const float4 c = s_acc(w, rn, e4);
                A.x += c.x * f; A.y += c.y * f; A.z += c.z * f; A.w += c.w * f;
            }
            const int64_t th = (int64_t)(r / hpg) * p.H + (g * hpg + r % hpg);
            if (nsplit == 1) {
                const float inv = L > 0.0f ? 1.0f / L : 0.0f;
                *reinterpret_cast<float4*>(p.out + th * DV + 4 * e4) =
                    make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
            } else {
                *reinterpret_cast<float4*>(ws_acc + (th * nsplit + sp) * DV + 4 * e4) = A;
                if (e4 == 0) {
                    ws_ml[(th * nsplit + sp) * 2 + 0] = M;
                    ws_ml[(th * nsplit + sp) * 2 + 1] = L;
                }
            }
        }
    }
}

template <int D, int DV, int NB, bool EPI>
hipError_t launch_t(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    auto kern = decode_mfma_kernel<D, DV, NB, EPI>;
    constexpr size_t lds = sizeof(float4) * kWaves * kTile * (D / 4 + DV / 4) + sizeof(float) * 2 * kWaves * 16;
    static bool configured = false;
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const dim3 grid = plan.k_new ? dim3((unsigned)(plan.splits * p.G)) : dim3((unsigned)plan.splits, (unsigned)p.G);
    return launch_kernel(kern, grid, dim3(kThreads), (uint32_t)lds, L, p, plan, ws);
}

template <int D, int DV, int NB>
hipError_t launch_nb(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    if (p.ep.any()) return launch_t<D, DV, NB, true>(p, plan, ws, L);
    return launch_t<D, DV, NB, false>(p, plan, ws, L);
}

template <int D, int DV>
hipError_t launch_dv(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    if (plan.nq <= 16) return launch_nb<D, DV, 1>(p, plan, ws, L);
    if constexpr (D <= 128) {
        if (plan.nq <= 32) return launch_nb<D, DV, 2>(p, plan, ws, L);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Query rows per KV group the matrix-core decode holds at (D, Dv): 16 per row
// block, two blocks up to headDim 128 (0: no instance).
int decode_mfma_max_rows(int D, int Dv) {
    if ((D == 64 && Dv == 64) || (D == 128 && Dv == 128)) return 32;
    if (D == 192 && Dv == 128) return 16;
    return 0;
}

hipError_t launch_decode_mfma(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    if (plan.splits < 1 || plan.splits > kMaxSplits) return hipErrorInvalidValue;
    if (p.ep.pb_weight || p.ep.rel_k) return hipErrorInvalidValue;  // no relative-position terms here
    if (plan.block > 0 && plan.block < kTile) return hipErrorInvalidValue;
    if (p.D == 64 && p.Dv == 64) return launch_dv<64, 64>(p, plan, ws, L);
    if (p.D == 128 && p.Dv == 128) return launch_dv<128, 128>(p, plan, ws, L);
    if (p.D == 192 && p.Dv == 128) return launch_dv<192, 128>(p, plan, ws, L);
    return hipErrorInvalidValue;
}

}  // namespace attn
