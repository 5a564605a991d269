// Decode path of op `attention`: few query rows against a long key/value
// range (a KV cache). HBM-bound: every visible K and V row of a KV head is
// read exactly once, for all the query rows of that head's group.
//
// decode_split: grid (splits, kv_heads), 256 threads (1-D on appending
// calls). The workgroup of KV head g walks its share of the key range. Its
// 256 lanes form 16 row groups of 16 lanes (one DPP row each); a row group
// takes U consecutive key rows at a time, and each lane of it loads a
// 4-float slice of every 64-float stretch of the K and V rows (128-bit
// loads, a whole row per 16 lanes). By default a lane holds one batch at a
// time: it uses the batch, then fetches the next (with more loads in flight
// per lane this memory system ran slower); a ring of 2 or 3 batches is an
// option. Dot products are partial per lane and summed across the row
// with DPP rotations, so every lane of the row group holds every score.
// The score epilogue and an online softmax follow, and the lane accumulates
// its V slice for all query rows of the group. At the end the 16 row
// groups' partial states are merged (lane shuffles, then LDS) into one
// (max, sum, acc) per query row and split. On an appending call one more
// split per KV head takes the call's new key and value rows straight from
// the caller's buffers and stores them into the caches as it reads them: a
// decode step needs no copy launch first.
//
// The running maximum is moved lazily: weights are taken against a
// reference that may trail the true maximum by up to 2^8 (so a weight is at
// most 256, far from f32 overflow), and the accumulator is rescaled only
// when a score passes the reference by more than that. Maxima live in the
// base-2 domain (scores times log2 e), so every exponential is one exp2.
//
// decode_combine: grid (T*heads), merges the splits' partial states:
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum acc_i 2^(m_i - M) / L.
// combine_few: the same merge for up to 16 splits of many rows (prefill
// key-range parts), one thread per 4 output floats.
#include "device_common.h"
#include "rope_device.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kRowGroups = kThreads / 16;
constexpr int kWaves = kThreads / 64;
constexpr float kLazy = 8.0f;  // log2 of the largest weight before the reference moves
constexpr int kMaxSplits = 1024;
constexpr int kFewSplits = 16;  // up to this many splits, combine_few_kernel merges them
constexpr int64_t kFewMinOutputs = 65536;  // ... when there are at least this many output float4s

template <int D, int DV, int NQ, bool EPI>
struct DecodeShape {
    // float4 per lane per K / V row: lane ln of a row group takes channels
    // 64 j + 4 ln .. + 3; past the width (80- or 96-wide rows: the second
    // group is partly empty) a lane loads the row's last float4 again, zeroes
    // it where it enters a product, and stores nothing.
    static constexpr int KJ = (D + 63) / 64;
    static constexpr int VJ = (DV + 63) / 64;
    // Key rows per row group per batch (one batch per lane at a time). Fewer
    // loads in flight ran faster, down to about four float4s per lane: with
    // 128-wide heads the epilogue-free instance takes one-row batches (4
    // loads; Llama-shaped decode 43.3 us against 45.5 us with two-row ones,
    // the 4096-window streaming decode 13.1 against 14.3), but the instances
    // with softcap, ALiBi, bias or relative-position terms are faster with
    // two-row batches (softcap 48.2 against 53.5 us; bucketed bias 48.5
    // against 58.7), and 64-wide heads (1 + 1 loads per row) need two rows
    // (49.2 against 64.8 us). Rows of 5 or more loads (192/128, 256) take
    // one. (Two-row batches also need q and acc, 4 NQ (KJ+VJ) registers, to
    // stay under ~170 registers with the ring.)
    static constexpr int U = (KJ + VJ) * 2 <= 8 && (KJ + VJ) * (16 + 4 * NQ) <= 170 && (EPI || KJ + VJ < 4) ? 2 : 1;
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// RM: the relative-position terms (bucketed position bias, relative
// key/value embeddings). 0: off. 1: on, for splits whose keys are all at the
// tables' far end for every row (their terms are per-row constants). 2: on,
// looked up per key (the split of keys near the query rows, the sink split,
// and non-causal calls). RM = 2 implies EPI.
// EPI: whether softcap, ALiBi or a bias can be on; without them the score
// is the scaled dot product and the code for the rest is left out (with
// RM = 1, plus the per-row constants of the far splits and, in the near
// split's loop, the relative-position terms, all in the scaled domain).
// DEPTH: batches of U rows per row group held in registers. 1 (the default):
// one batch at a time, the next fetched once the current one is used; 2 or
// 3: a ring, DEPTH-1 batches in flight while one is used.
template <int D, int DV, int NQ, bool EPI, int RM, int DEPTH>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(Problem p, DecodePlan plan,
                                                                   float* __restrict__ ws) {
    using Sh = DecodeShape<D, DV, NQ, EPI>;
    constexpr int KJ = Sh::KJ, VJ = Sh::VJ, U = Sh::U;
    constexpr int kStep = kRowGroups * U;

    const int tid = threadIdx.x;
    const int ln = tid & 15;
    const int rg = tid >> 4;
    // Whether this lane's float4 j of a K / V row lies within the row, and the
    // in-row offset it loads from (the row's last float4 when it does not).
    auto kin = [&](int j) { return 64 * j + 64 <= D || 64 * j + 4 * ln < D; };
    auto vin = [&](int j) { return 64 * j + 64 <= DV || 64 * j + 4 * ln < DV; };
    auto koff = [&](int j) { return kin(j) ? 64 * j : D - 4 - 4 * ln; };
    auto voff = [&](int j) { return vin(j) ? 64 * j : DV - 4 - 4 * ln; };
    constexpr bool REL = RM != 0;
    constexpr bool FAR = RM == 1;
    // Split sp of KV group g. On an appending call the splits of appended
    // rows (short ones) are dispatched after every other workgroup: placed
    // first, they would push a third full-length split onto some CUs.
    int sp, g;
    if (plan.k_new) {
        const int per = plan.splits - 1;  // the other splits of a group
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

    // Query rows of this KV group: row r is query row t = r / hpg of head
    // h = g*hpg + r % hpg. Rows past nrows are padding and never written.
    float4 qr[NQ][KJ];
    int pos[NQ];
    int hh[NQ];
    int tt[NQ];
    bool live[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        live[r] = r < nrows;
        tt[r] = live[r] ? r / hpg : 0;
        hh[r] = g * hpg + (live[r] ? r % hpg : 0);
        pos[r] = p.ep.pos_offset + tt[r];
    }
    float slope[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) slope[r] = alibi_slope(p.ep, hh[r]);
    // With a rotary embedding, the raw q channels this thread turns, their pair
    // partners and frequencies are fetched first, ahead of the K/V loads.
    constexpr int QE = (NQ * D + kThreads - 1) / kThreads;
    float qa[QE], qb[QE], qf[QE];
#pragma unroll
    for (int c = 0; c < QE; ++c) {
        qa[c] = 0.0f;
        qb[c] = 0.0f;
        qf[c] = 0.0f;
    }
    if (p.rope.on) {
#pragma unroll
        for (int c = 0; c < QE; ++c) {
            const int e = tid + c * kThreads;
            const int r = e / D, d = e % D;
            if (e < NQ * D && r < nrows) {
                const int t = r / hpg, h = g * hpg + r % hpg;
                const float* head = p.q + (int64_t)t * p.H * D + (int64_t)h * D;
                const RopeTap tp = rope_tap(p.rope, d);
                qa[c] = head[d];
                qb[c] = head[tp.partner];
                qf[c] = p.rope.inv_freq[tp.i];
            }
        }
    }
    float m[NQ], l[NQ];
    float4 acc[NQ][VJ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
#pragma unroll
        for (int j = 0; j < VJ; ++j) acc[r][j] = zero4();
    }

    // This split's keys: its share of the window range, or (the last split,
    // with attention sinks) the sink keys below it.
    // (With relative-position terms, the split before it covers the keys
    // near the query rows; on an appending call, the rows appended.)
    const bool sink_split = plan.sink_hi > 0 && sp == plan.splits - 1;
    const bool near_split = plan.near_hi > plan.near_lo && sp == plan.splits - 1 - (plan.sink_hi > 0 ? 1 : 0);
    // The appended rows come from the caller's new-row buffers, and this
    // split also stores them into the caches (no other split reads them).
    const bool append = !REL && near_split && plan.k_new != nullptr;
    const bool spread = plan.block > 0 && !sink_split && !near_split;
    // [k0, k1): the rows the split's keys lie in. A split walks nw rows in
    // blocks of 2^bsh; its j-th block is block (j * bstride + boff) of
    // [k0, k1), less bwrap when that passes bwrap.
    int k0, k1, nw, bsh, bstride = 1, boff = 0, bwrap = INT_MAX;
    if (spread) {
        // Splits of the range interleave blocks: at any moment every split
        // reads near every other, so all of them see the same mix of memory
        // channels instead of each camping on its own stretch.
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
        bsh = 31 - __builtin_clz((unsigned)kStep);
        // A chunk may be walked from a rotated start (a whole number of
        // batch steps), so that splits whose chunks start at aligned
        // addresses do not all hit the same memory channels at once.
        if (plan.rotate > 0 && nw > 0 && nw % kStep == 0) {
            boff = (int)((((int64_t)sp * plan.rotate) % nw) >> bsh);
            bwrap = nw >> bsh;
        }
    }
    // The walk goes in steps of kStep rows, one batch of U rows per row
    // group; a step never straddles a block. First row of step st (the same
    // for the whole workgroup, so it stays in scalar registers):
    auto step_row = [&](int st) {
        const int w = st * kStep;
        int b = (w >> bsh) * bstride + boff;
        if (b >= bwrap) b -= bwrap;
        return k0 + (b << bsh) + (w & ((1 << bsh) - 1));
    };
    const int w_rg = rg * U;  // this row group's batch within a step
    const int nsteps = (nw + kStep - 1) / kStep;
    // Workgroup-uniform bases; per-lane offsets stay in 32 bits (the host
    // keeps (k1 - k0) * row stride below 2^31 floats).
    const uint32_t kstride = (uint32_t)(p.G * D), vstride = (uint32_t)(p.G * DV);
    const float* kwg = (append ? plan.k_new : p.k + (int64_t)k0 * kstride) + (int64_t)g * D + 4 * ln;
    const float* vwg = (append ? plan.v_new : p.v + (int64_t)k0 * vstride) + (int64_t)g * DV + 4 * ln;
    // With every key of [k0, k1) visible to every row, only rows past the
    // walk's or the range's end need checking.
    const bool dense = chunk_all_visible(p.ep, p.ep.pos_offset, p.ep.pos_offset + (int)p.T - 1, k0, k1);
    // Relative key/value embeddings: every row's products with every key
    // embedding go to LDS once q is in registers. A split whose keys all lie
    // max_distance or more before the first row's position uses embedding 0
    // alone: a per-row constant in the scores and l * rel_v[0] in the sums.
    const bool rel = REL && p.ep.rel_k != nullptr;
    const int nrel = rel ? 2 * p.ep.rel_max + 1 : 0;
    const bool rel_far = rel && k1 - 1 <= p.ep.pos_offset - p.ep.rel_max;
    // Likewise a split whose keys all lie at least the last threshold before
    // the first row takes the last bucket's bias for every key: one number per row.
    const bool pb = REL && p.ep.pb_weight != nullptr;
    const bool pb_far = pb && k1 - 1 <= p.ep.pos_offset - p.ep.pb_dt;
    // FAR instances run far splits through the batched walk with those
    // constants, and a split of keys near the rows through a plain loop, one
    // key per row group at a time, with every term looked up per key.
    const bool split_far = (!pb || pb_far) && (!rel || rel_far);
    const bool near_loop = FAR && !split_far;
    float pbc[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        pbc[r] = 0.0f;
        if (pb_far) pbc[r] = p.ep.pb_weight[(p.ep.pb_n - 1) * p.ep.pb_heads + hh[r]];
    }
    // [NQ][nrel], then the position-bias bucket of each distance, then (from
    // a 4-byte boundary) each row's weight of each bucket, [buckets][NQ].
    extern __shared__ float s_qrel[];
    uint8_t* s_pbb = reinterpret_cast<uint8_t*>(s_qrel + NQ * nrel);
    float* s_pbw = reinterpret_cast<float*>(s_pbb + ((p.ep.pb_dt + 3) & ~3));
    float qrel0[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) qrel0[r] = 0.0f;

    if constexpr (REL) {
        // The bucket of each distance, copied to LDS for per-key lookups
        // (before any batch is fetched: the fetches look buckets up).
        if (pb && !(FAR && split_far)) {
            for (int d = tid; d < p.ep.pb_dt; d += kThreads) s_pbb[d] = p.ep.pb_bucket[d];
            // The weights too: a per-key lookup is then two LDS reads, not an
            // LDS read and a dependent memory round trip per row.
            const int nbw = (p.ep.pb_bidir ? 2 : 1) * p.ep.pb_n * NQ;
            for (int i = tid; i < nbw; i += kThreads) {
                const int b = i / NQ, r = i - b * NQ;
                s_pbw[i] = p.ep.pb_weight[b * p.ep.pb_heads + g * hpg + (r < nrows ? r % hpg : 0)];
            }
            __syncthreads();
        }
    }

    // Rows past the walk's or the range's end are clamped to row k1 - 1 (in
    // bounds) and their scores masked, so the loads need no branches. The bias entries of
    // a batch travel with its K/V rows, so their latency is hidden too.
    constexpr int BR = EPI ? NQ : 1;
    auto load = [&](float4 (&kf)[U][KJ], float4 (&vf)[U][VJ], float (&bf)[BR][U], int st) {
        const int r0 = step_row(st) + w_rg;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sc = min(r0 + u, k1 - 1);
            const uint32_t row = (uint32_t)(sc - k0);
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const float4 x = load_stream4(kwg + row * kstride + koff(j));
                kf[u][j] = kin(j) ? x : zero4();
            }
#pragma unroll
            for (int j = 0; j < VJ; ++j) vf[u][j] = load_stream4(vwg + row * vstride + voff(j));
            if constexpr (EPI) {
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    float b = 0.0f;
                    if (p.ep.bias_kind == ATTN_BIAS_TS) b = p.bias[(int64_t)tt[r] * p.S + sc];
                    else if (p.ep.bias_kind == ATTN_BIAS_HTS)
                        b = p.bias[((int64_t)hh[r] * p.T + tt[r]) * p.S + sc];
                    if constexpr (REL) {
                        if constexpr (FAR) b += pbc[r];
                        else if (pb_far) b += pbc[r];
                        else if (pb) b += pb_row_tab_n<NQ>(p.ep, s_pbb, s_pbw, r, pos[r], sc);
                    }
                    bf[r][u] = b;
                }
            }
        }
    };

    auto process = [&](const float4 (&kf)[U][KJ], const float4 (&vf)[U][VJ], const float (&bf)[BR][U],
                       int st) {
        const int w0 = st * kStep + w_rg;
        const int r0 = step_row(st) + w_rg;
        // Rows to mask only past the walk's or the range's end, or where not
        // every row sees every key; the masks are worked out only when some
        // lane of the wave has such rows.
        const bool check = !(dense && w0 + U <= nw && r0 + U <= k1);
        float x[NQ][U];
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = 0.0f;
#pragma unroll
                for (int j = 0; j < KJ; ++j) dot = dot4(qr[r][j], kf[u][j], dot);
                dot = row16_sum(dot);
                const int s = r0 + u;
                if constexpr (REL) {
                    if constexpr (FAR) dot += qrel0[r];
                    else if (rel_far) dot += qrel0[r];
                    else if (rel) dot += s_qrel[r * nrel + rel_row(p.ep, pos[r], s)];
                }
                if constexpr (EPI) {
                    x[r][u] = score_epilogue(dot, p.ep, slope[r], pos[r], s, bf[r][u]) * kLog2e;
                } else {
                    x[r][u] = dot;  // q carries scale * log2(e)
                }
            }
        }
        if (__ballot(check)) {
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int s = r0 + u;
                    const bool vis = !check | (live[r] & (w0 + u < nw) & (s < k1) & key_visible(p.ep, pos[r], s));
                    if (!vis) x[r][u] = -INFINITY;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            float mx = x[r][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, x[r][u]);
            if (mx > m[r] + kLazy) {
                const float alpha = fast_exp2(m[r] - mx);
                l[r] *= alpha;
#pragma unroll
                for (int j = 0; j < VJ; ++j) {
                    acc[r][j].x *= alpha; acc[r][j].y *= alpha;
                    acc[r][j].z *= alpha; acc[r][j].w *= alpha;
                }
                m[r] = mx;
            }
            const float mu = m[r] == -INFINITY ? 0.0f : m[r];
            float pu[U];
            float psum = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[u] = fast_exp2(x[r][u] - mu);
                psum += pu[u];
            }
            l[r] += psum;
#pragma unroll
            for (int j = 0; j < VJ; ++j) {
                float4 a = acc[r][j];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    a.x = fmaf(pu[u], vf[u][j].x, a.x);
                    a.y = fmaf(pu[u], vf[u][j].y, a.y);
                    a.z = fmaf(pu[u], vf[u][j].z, a.z);
                    a.w = fmaf(pu[u], vf[u][j].w, a.w);
                }
                acc[r][j] = a;
            }
            if constexpr (REL && !FAR) {
                if (rel && !rel_far && p.ep.rel_v) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const float* rv = p.ep.rel_v + (int64_t)rel_row(p.ep, pos[r], r0 + u) * DV + 4 * ln;
#pragma unroll
                        for (int j = 0; j < VJ; ++j) {
                            const float4 x4 = ld4(rv + voff(j));
                            acc[r][j].x = fmaf(pu[u], x4.x, acc[r][j].x);
                            acc[r][j].y = fmaf(pu[u], x4.y, acc[r][j].y);
                            acc[r][j].z = fmaf(pu[u], x4.z, acc[r][j].z);
                            acc[r][j].w = fmaf(pu[u], x4.w, acc[r][j].w);
                        }
                    }
                }
            }
        }
        if constexpr (!REL) {
            // Rows read from the new-row buffers go on into the caches: each
            // lane stores the slices it loaded.
            // (Uniform bases and 32-bit lane offsets, so that no per-lane
            // address stays live through the walk.)
            if (append) {
                float* kd = plan.k_cache + (int64_t)k0 * kstride + (int64_t)g * D;
                float* vd = plan.v_cache + (int64_t)k0 * vstride + (int64_t)g * DV;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (w0 + u < nw && r0 + u < k1) {
                        const uint32_t row = (uint32_t)(r0 + u - k0);
#pragma unroll
                        for (int j = 0; j < KJ; ++j)
                            if (kin(j)) *reinterpret_cast<float4*>(kd + (row * kstride + 4 * ln + 64 * j)) = kf[u][j];
#pragma unroll
                        for (int j = 0; j < VJ; ++j)
                            if (vin(j)) *reinterpret_cast<float4*>(vd + (row * vstride + 4 * ln + 64 * j)) = vf[u][j];
                    }
                }
            }
        }
    };

    {
        // DEPTH batch slots: one (a batch at a time) or a ring in which
        // batch i of a round is used while batches i+1 .. i+DEPTH-1 are in
        // flight. The epilogue-free far walk of the relative-position
        // instances keeps two slots at DEPTH 1 (below).
        constexpr int kSlots = DEPTH > 1 ? DEPTH : FAR && !EPI ? 2 : 1;
        float4 kr[kSlots][U][KJ], vr[kSlots][U][VJ];
        float br[kSlots][BR][U];
        // In a ring (DEPTH >= 2) with the epilogue on, batches are prefetched
        // unconditionally (load() clamps rows past the chunk's end, so one
        // spare batch is read at the end): a conditional load makes the
        // compiler's wait counts assume it was skipped, so processing a batch
        // would also wait for most of the next one. Measured on the
        // latent-shaped ALiBi+bias decode: 31.6 -> 30.6 us. Without the
        // epilogue the spare batch's latency at the end costs more than the
        // overlap gains (46.4 -> 47.0 us on the Llama-shaped decode), so
        // those instances keep the condition. (With one batch at a time, the
        // default, there is no overlap to lose.)
        constexpr bool kAlwaysPrefetch = EPI;
        // The first batch (the first DEPTH-1 of a ring) is on its way before
        // q is fetched and set up, so its latency overlaps that work.
        constexpr int kLead = DEPTH > 1 ? DEPTH - 1 : 1;
#pragma unroll
        for (int i = 0; i < kLead; ++i)
            if (!near_loop && (kAlwaysPrefetch || i < nsteps)) load(kr[i], vr[i], br[i], i);
        // q is loaded (and turned, with a rotary embedding) while the first
        // K/V batches are in flight.
        if (p.rope.on) {
            // Every row group needs the same turned q, so each workgroup turns
            // it once, through LDS: the raw channels were fetched before the
            // K/V batches were issued, the turn happens while those load.
            __shared__ __align__(16) float s_q[NQ * D];
#pragma unroll
            for (int c = 0; c < QE; ++c) {
                const int e = tid + c * kThreads;
                if (e < NQ * D) {
                    const int r = e / D, d = e % D;
                    const int t = r / hpg;
                    s_q[e] = r < nrows ? rope_turn(p.rope, rope_tap(p.rope, d), qa[c], qb[c], qf[c], p.rope.pos0 + t)
                                       : 0.0f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < NQ; ++r)
#pragma unroll
                for (int j = 0; j < KJ; ++j)
                    qr[r][j] = kin(j) ? *reinterpret_cast<const float4*>(s_q + r * D + 64 * j + 4 * ln) : zero4();
        } else {
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float* qrow = p.q + (int64_t)tt[r] * p.H * D + (int64_t)hh[r] * D + 4 * ln;
#pragma unroll
                for (int j = 0; j < KJ; ++j) qr[r][j] = live[r] && kin(j) ? ld4(qrow + 64 * j) : zero4();
            }
        }
        if constexpr (!EPI) {
            // Without an epilogue the score is the scaled product: q takes
            // the scale (and the base change of exp2) once.
            const float c = p.ep.scale * kLog2e;
#pragma unroll
            for (int r = 0; r < NQ; ++r)
#pragma unroll
                for (int j = 0; j < KJ; ++j) {
                    qr[r][j].x *= c; qr[r][j].y *= c; qr[r][j].z *= c; qr[r][j].w *= c;
                }
        }
        if constexpr (REL) {
            if (rel && FAR && split_far) {
                // Far keys all take embedding 0: one product per row, summed
                // across the row group's 16 lanes (every lane gets it).
                float4 kv[KJ];
#pragma unroll
                for (int jj = 0; jj < KJ; ++jj) kv[jj] = ld4(p.ep.rel_k + 4 * ln + koff(jj));
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    float d = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < KJ; ++jj) d = dot4(qr[r][jj], kv[jj], d);
                    qrel0[r] = row16_sum(d);
                }
            } else if (rel) {
                // q . rel_k[j] per row: row group rg takes j = rg, rg + 16, ...,
                // four embeddings' loads in flight at a time.
                for (int j0 = rg; j0 < nrel; j0 += 4 * kRowGroups) {
                    float4 kv[4][KJ];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = min(j0 + i * kRowGroups, nrel - 1);
#pragma unroll
                        for (int jj = 0; jj < KJ; ++jj) kv[i][jj] = ld4(p.ep.rel_k + (int64_t)j * D + 4 * ln + koff(jj));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = j0 + i * kRowGroups;
#pragma unroll
                        for (int r = 0; r < NQ; ++r) {
                            float d = 0.0f;
#pragma unroll
                            for (int jj = 0; jj < KJ; ++jj) d = dot4(qr[r][jj], kv[i][jj], d);
                            d = row16_sum(d);
                            if (ln == 0 && j < nrel) s_qrel[r * nrel + j] = d;
                        }
                    }
                }
            }
            if (!(FAR && split_far) && rel) {
                __syncthreads();
#pragma unroll
                for (int r = 0; r < NQ; ++r) qrel0[r] = rel ? s_qrel[r * nrel] : 0.0f;
            }
            if constexpr (FAR && !EPI) {
                // No other epilogue term: a far split's scores are the scaled
                // product (q carries scale * log2(e)) plus one constant per
                // row in the same base-2 domain, the embedding-0 product
                // (formed with the scaled q) and the last bucket's bias.
                if (split_far) {
#pragma unroll
                    for (int r = 0; r < NQ; ++r) qrel0[r] += pbc[r] * kLog2e;
                }
            }
        }
        if constexpr (FAR) {
            if (near_loop) {
                // Keys near the rows: one key per row group at a time, every
                // relative-position term looked up (LDS tables), v + rel_v[j].
                for (int s = k0 + rg; s < k1; s += kRowGroups) {
                    const uint32_t row = (uint32_t)(s - k0);
                    float4 kf[KJ], vf[VJ];
#pragma unroll
                    for (int j = 0; j < KJ; ++j) kf[j] = kin(j) ? ld4(kwg + row * kstride + koff(j)) : zero4();
#pragma unroll
                    for (int j = 0; j < VJ; ++j) vf[j] = ld4(vwg + row * vstride + voff(j));
                    // Each row's relative value embedding, requested with the
                    // key's K and V rows (requested after the row's softmax,
                    // each was a dependent round trip: the near split then
                    // outlasted the far ones, Llama-shaped decode with
                    // relative keys/values 47.9 -> 46.2 us). Eight-row
                    // instances keep one shared row, which serves every row
                    // of a one-query call (all rows at one position); with
                    // more query rows they load per row as the row needs it.
                    constexpr int NRV = NQ > 4 ? 1 : NQ;
                    const bool rv_early = rel && p.ep.rel_v && (NQ <= 4 || p.T == 1);
                    float4 rvr[NRV][VJ];
#pragma unroll
                    for (int r = 0; r < NRV; ++r)
#pragma unroll
                        for (int j = 0; j < VJ; ++j)
                            rvr[r][j] = rv_early
                                            ? ld4(p.ep.rel_v + (int64_t)rel_row(p.ep, pos[r], s) * DV + 4 * ln + voff(j))
                                            : zero4();
#pragma unroll
                    for (int r = 0; r < NQ; ++r) {
                        float dot = 0.0f;
#pragma unroll
                        for (int j = 0; j < KJ; ++j) dot = dot4(qr[r][j], kf[j], dot);
                        dot = row16_sum(dot);
                        const int jr = rel ? rel_row(p.ep, pos[r], s) : 0;
                        if (rel) dot += s_qrel[r * nrel + jr];
                        float b = 0.0f;
                        if (p.ep.bias_kind == ATTN_BIAS_TS) b = p.bias[(int64_t)tt[r] * p.S + s];
                        else if (p.ep.bias_kind == ATTN_BIAS_HTS) b = p.bias[((int64_t)hh[r] * p.T + tt[r]) * p.S + s];
                        if (pb) b += pb_row_tab_n<NQ>(p.ep, s_pbb, s_pbw, r, pos[r], s);
                        float xs;
                        if constexpr (EPI) xs = score_epilogue(dot, p.ep, slope[r], pos[r], s, b) * kLog2e;
                        else xs = dot + b * kLog2e;  // scaled q and embedding products; b: the position bias
                        xs = (live[r] & key_visible(p.ep, pos[r], s)) ? xs : -INFINITY;
                        if (xs > m[r] + kLazy) {
                            const float alpha = fast_exp2(m[r] - xs);
                            l[r] *= alpha;
#pragma unroll
                            for (int j = 0; j < VJ; ++j) {
                                acc[r][j].x *= alpha; acc[r][j].y *= alpha;
                                acc[r][j].z *= alpha; acc[r][j].w *= alpha;
                            }
                            m[r] = xs;
                        }
                        const float pw = fast_exp2(xs - (m[r] == -INFINITY ? 0.0f : m[r]));
                        l[r] += pw;
#pragma unroll
                        for (int j = 0; j < VJ; ++j) {
                            float4 vv = vf[j];
                            float4 rv = rvr[NRV > 1 ? r : 0][j];
                            if (NQ > 4 && !rv_early && rel && p.ep.rel_v)
                                rv = ld4(p.ep.rel_v + (int64_t)jr * DV + 4 * ln + voff(j));
                            vv.x += rv.x; vv.y += rv.y; vv.z += rv.z; vv.w += rv.w;
                            acc[r][j].x = fmaf(pw, vv.x, acc[r][j].x);
                            acc[r][j].y = fmaf(pw, vv.y, acc[r][j].y);
                            acc[r][j].z = fmaf(pw, vv.z, acc[r][j].z);
                            acc[r][j].w = fmaf(pw, vv.w, acc[r][j].w);
                        }
                    }
                }
            }
        }
        bool done = near_loop;
        if constexpr (DEPTH == 1 && FAR && !EPI) {
            // Far splits of the epilogue-free relative-position instance:
            // still one batch in flight per lane, but the next one is
            // requested as soon as the current one has arrived, before it is
            // used (the two slots in turn; the wait drains this lane's only
            // batch in flight). Llama-shaped decode, one box, two or three
            // rounds: T5 bias 45.6-45.7 -> 44.5 us, relative keys/values
            // 46.1-46.2 -> 45.1 us. The same walk measured 0.3 us slower on
            // the plain decode, which keeps the loop below.
            for (int st = 0; st < nsteps && !done; st += 2) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (st + 1 < nsteps) load(kr[1], vr[1], br[1], st + 1);
                __builtin_amdgcn_sched_barrier(0);
                process(kr[0], vr[0], br[0], st);
                if (st + 1 >= nsteps) break;
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (st + 2 < nsteps) load(kr[0], vr[0], br[0], st + 2);
                __builtin_amdgcn_sched_barrier(0);
                process(kr[1], vr[1], br[1], st + 1);
            }
            done = true;
        }
        if constexpr (DEPTH == 1) {
            // One batch per lane at a time: use it, then fetch the next into
            // the same registers.
            for (int st = 0; st < nsteps && !done; ++st) {
                process(kr[0], vr[0], br[0], st);
                if (st + 1 < nsteps) load(kr[0], vr[0], br[0], st + 1);
            }
            done = true;
        }
        for (int st = 0; st < nsteps && !done; st += DEPTH) {
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                const int sn = st + i + DEPTH - 1;
                const int nx = (i + DEPTH - 1) % DEPTH;  // a constant once unrolled
                if (kAlwaysPrefetch || sn < nsteps) load(kr[nx], vr[nx], br[nx], sn);
                if (st + i >= nsteps) {
                    done = true;
                    break;
                }
                process(kr[i], vr[i], br[i], st + i);
            }
        }
    }

    if constexpr (REL) {
        // A far split's keys all take rel_v[0]: add it once, weighted by l.
        if (rel_far && p.ep.rel_v) {
#pragma unroll
            for (int r = 0; r < NQ; ++r)
#pragma unroll
                for (int j = 0; j < VJ; ++j) {
                    const float4 x4 = ld4(p.ep.rel_v + 4 * ln + voff(j));
                    acc[r][j].x = fmaf(l[r], x4.x, acc[r][j].x);
                    acc[r][j].y = fmaf(l[r], x4.y, acc[r][j].y);
                    acc[r][j].z = fmaf(l[r], x4.z, acc[r][j].z);
                    acc[r][j].w = fmaf(l[r], x4.w, acc[r][j].w);
                }
        }
    }

    // Merge the four row groups of each wave (lanes 16 and 32 apart hold the
    // same V slice of another row group).
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const float mo = __shfl_xor(m[r], off, 64);
            const float lo = __shfl_xor(l[r], off, 64);
            const float M = fmaxf(m[r], mo);
            const float Mu = M == -INFINITY ? 0.0f : M;
            const float a = fast_exp2(m[r] - Mu), b = fast_exp2(mo - Mu);
            l[r] = l[r] * a + lo * b;
            m[r] = M;
#pragma unroll
            for (int j = 0; j < VJ; ++j) {
                float4& c = acc[r][j];
                c.x = c.x * a + __shfl_xor(c.x, off, 64) * b;
                c.y = c.y * a + __shfl_xor(c.y, off, 64) * b;
                c.z = c.z * a + __shfl_xor(c.z, off, 64) * b;
                c.w = c.w * a + __shfl_xor(c.w, off, 64) * b;
            }
        }
    }

    // Then the four waves, through LDS.
    __shared__ float s_m[kWaves][NQ], s_l[kWaves][NQ];
    __shared__ float4 s_acc[kWaves][NQ][DV / 4];
    const int wave = tid >> 6;
    if ((tid & 63) < 16) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            if (ln == 0) {
                s_m[wave][r] = m[r];
                s_l[wave][r] = l[r];
            }
#pragma unroll
            for (int j = 0; j < VJ; ++j)
                if (vin(j)) s_acc[wave][r][j * 16 + ln] = acc[r][j];
        }
    }
    __syncthreads();

    const int nsplit = plan.splits;
    float* ws_acc = ws;
    float* ws_ml = ws + (int64_t)p.T * p.H * nsplit * DV;
    for (int idx = tid; idx < NQ * (DV / 4); idx += kThreads) {
        const int r = idx / (DV / 4), e4 = idx % (DV / 4);
        if (r >= nrows) continue;
        float M = s_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
        const float Mu = M == -INFINITY ? 0.0f : M;
        float L = 0.0f;
        float4 A = zero4();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(s_m[w][r] - Mu);
            L += s_l[w][r] * f;
            const float4 c = s_acc[w][r][e4];
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

// One workgroup per (query row, head). Thread group grp (E4 threads, one
// float4 column each) takes splits grp, grp + kGroups, ...: it merges their
// (max, sum, acc) on its own, from loads all requested up front, and one
// barrier later the first group merges the groups' results.
template <int DV>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(Problem p, int nsplit,
                                                                  const float* __restrict__ ws) {
    constexpr int E4 = DV / 4;
    constexpr int kGroups = kThreads / E4;
    // Up-front loads cover 64 splits of the key range plus the near and sink
    // splits; further splits (plans with few KV heads) are read afterwards.
    constexpr int kPreSplits = 66;
    constexpr int kPre = (kPreSplits + kGroups - 1) / kGroups;
    __shared__ float2 s_ml[kGroups];
    __shared__ float4 s_part[kGroups][E4];

    const int tid = threadIdx.x;
    const int e4 = tid % E4, grp = tid / E4;
    // With E4 not dividing the workgroup (80- and 96-wide rows) the last
    // threads form no whole group: they only keep the barrier.
    const bool active = grp < kGroups;
    const int64_t th = blockIdx.x;  // t * H + h
    const float4* acc4 = reinterpret_cast<const float4*>(ws + th * nsplit * DV);
    const float2* ml2 = reinterpret_cast<const float2*>(ws + (int64_t)p.T * p.H * nsplit * DV + th * nsplit * 2);
    float4* orow = reinterpret_cast<float4*>(p.out + th * DV);

    float4 pre[kPre];
    float2 mlp[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int i = active ? grp + u * kGroups : nsplit;
        pre[u] = i < nsplit ? acc4[(int64_t)i * E4 + e4] : zero4();
        mlp[u] = i < nsplit ? ml2[i] : make_float2(-INFINITY, 0.0f);
    }
    // The group's maximum, then its sum and accumulator against it; splits
    // past the up-front loads come in chunks of kChunk per group (all their
    // loads in flight at once), merged into the running state as they arrive.
    float mg = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPre; ++u) mg = fmaxf(mg, mlp[u].x);
    float lg = 0.0f;
    float4 a = zero4();
    {
        const float mu = mg == -INFINITY ? 0.0f : mg;
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const float w = fast_exp2(mlp[u].x - mu);
            lg = fmaf(mlp[u].y, w, lg);
            a.x = fmaf(pre[u].x, w, a.x); a.y = fmaf(pre[u].y, w, a.y);
            a.z = fmaf(pre[u].z, w, a.z); a.w = fmaf(pre[u].w, w, a.w);
        }
    }
    constexpr int kChunk = 16;
    const int i_rest = active ? grp + kPre * kGroups : nsplit;  // splits past the up-front loads
    for (int i0 = i_rest; i0 < nsplit; i0 += kChunk * kGroups) {
        float2 mc[kChunk];
        float4 cc[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int i = i0 + u * kGroups;
            mc[u] = i < nsplit ? ml2[i] : make_float2(-INFINITY, 0.0f);
            cc[u] = i < nsplit ? acc4[(int64_t)i * E4 + e4] : zero4();
        }
        float mx = mg;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) mx = fmaxf(mx, mc[u].x);
        const float mu = mx == -INFINITY ? 0.0f : mx;
        const float r = fast_exp2(mg - mu);  // 0 while nothing is merged yet
        lg *= r;
        a.x *= r; a.y *= r; a.z *= r; a.w *= r;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float w = fast_exp2(mc[u].x - mu);
            lg = fmaf(mc[u].y, w, lg);
            a.x = fmaf(cc[u].x, w, a.x); a.y = fmaf(cc[u].y, w, a.y);
            a.z = fmaf(cc[u].z, w, a.z); a.w = fmaf(cc[u].w, w, a.w);
        }
        mg = mx;
    }
    if (active) {
        s_part[grp][e4] = a;
        if (e4 == 0) s_ml[grp] = make_float2(mg, lg);
    }
    __syncthreads();
    if (grp == 0) {
        float M = s_ml[0].x;
#pragma unroll
        for (int q = 1; q < kGroups; ++q) M = fmaxf(M, s_ml[q].x);
        if (M == -INFINITY) {  // no visible key in any split
            orow[e4] = zero4();
            return;
        }
        float L = 0.0f;
        float4 t = zero4();
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const float w = fast_exp2(s_ml[q].x - M);
            L = fmaf(s_ml[q].y, w, L);
            const float4 c = s_part[q][e4];
            t.x = fmaf(c.x, w, t.x); t.y = fmaf(c.y, w, t.y);
            t.z = fmaf(c.z, w, t.z); t.w = fmaf(c.w, w, t.w);
        }
        const float inv = 1.0f / L;
        orow[e4] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    }
}

// Few splits (key-range parts of a prefill): one thread per (query row,
// head, 4 output floats) reads every split's (max, sum) itself and its four
// accumulator floats; no reduction across threads is needed.
template <int DV>
__global__ __launch_bounds__(kThreads) void combine_few_kernel(Problem p, int nsplit,
                                                               const float* __restrict__ ws) {
    constexpr int E4 = DV / 4;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t rows = p.T * p.H;
    if (idx >= rows * E4) return;
    const int64_t th = idx / E4;
    const int e4 = (int)(idx % E4);
    const float* ml = ws + rows * nsplit * DV + th * nsplit * 2;
    const float4* acc4 = reinterpret_cast<const float4*>(ws + th * nsplit * DV) + e4;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[2 * i]);
    float4* orow = reinterpret_cast<float4*>(p.out + th * DV) + e4;
    if (M == -INFINITY) {
        *orow = zero4();
        return;
    }
    float L = 0.0f;
    float4 a = zero4();
    for (int i = 0; i < nsplit; ++i) {
        const float w = fast_exp2(ml[2 * i] - M);
        L = fmaf(ml[2 * i + 1], w, L);
        const float4 c = acc4[(int64_t)i * E4];
        a.x = fmaf(c.x, w, a.x); a.y = fmaf(c.y, w, a.y);
        a.z = fmaf(c.z, w, a.z); a.w = fmaf(c.w, w, a.w);
    }
    const float inv = 1.0f / L;
    *orow = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
}

template <int D, int DV, int NQ, int DEPTH>
hipError_t launch_split_d(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    const dim3 grid = plan.k_new ? dim3((unsigned)(plan.splits * p.G)) : dim3((unsigned)plan.splits, (unsigned)p.G);
    const bool epi = p.ep.any();
    // With relative embeddings, every row's products with them sit in LDS.
    const uint32_t lds = p.ep.rel_k ? (uint32_t)(sizeof(float) * NQ * (2 * p.ep.rel_max + 1)) : 0u;
    if (p.ep.pb_weight || p.ep.rel_k) {
        // Causal calls with a split of near keys: the far instance (batched
        // walk for far splits, plain loop for the near one); otherwise every
        // split looks its terms up per key.
        const uint32_t lds_all =
            lds + (p.ep.pb_weight ? (uint32_t)((p.ep.pb_dt + 3) & ~3) +
                                        (uint32_t)(sizeof(float) * NQ * (p.ep.pb_bidir ? 2 : 1) * p.ep.pb_n)
                                  : 0u);
        if (plan.near_hi > plan.near_lo) {
            // Without softcap, ALiBi or a bias input the far splits run the
            // epilogue-free walk (their terms are per-row constants).
            const bool other = p.ep.softcap > 0.0f || p.ep.has_alibi || p.ep.bias_kind != ATTN_BIAS_NONE;
            if (!other)
                return launch_kernel(decode_split_kernel<D, DV, NQ, false, 1, DEPTH>, grid, dim3(kThreads), lds_all,
                                     L, p, plan, ws);
            return launch_kernel(decode_split_kernel<D, DV, NQ, true, 1, DEPTH>, grid, dim3(kThreads), lds_all, L,
                                 p, plan, ws);
        }
        return launch_kernel(decode_split_kernel<D, DV, NQ, true, 2, DEPTH>, grid, dim3(kThreads), lds_all, L, p,
                             plan, ws);
    }
    if (epi) return launch_kernel(decode_split_kernel<D, DV, NQ, true, 0, DEPTH>, grid, dim3(kThreads), 0, L, p, plan, ws);
    return launch_kernel(decode_split_kernel<D, DV, NQ, false, 0, DEPTH>, grid, dim3(kThreads), 0, L, p, plan, ws);
}

// A third ring batch only where it fits beside q and acc without spilling:
// (KJ+VJ) * (24 + 4 NQ) registers for the ring, q and acc, under 200.
template <int D, int DV, int NQ>
constexpr bool depth3_fits() {
    return ((D + 63) / 64 + (DV + 63) / 64) * (24 + 4 * NQ) < 200;
}

template <int D, int DV, int NQ>
hipError_t launch_split_t(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    if constexpr (depth3_fits<D, DV, NQ>()) {
        if (plan.depth >= 3) return launch_split_d<D, DV, NQ, 3>(p, plan, ws, L);
    }
    if (plan.depth == 1) return launch_split_d<D, DV, NQ, 1>(p, plan, ws, L);
    return launch_split_d<D, DV, NQ, 2>(p, plan, ws, L);
}

template <int D, int DV>
hipError_t launch_split_nq(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    constexpr int KV = (D + 63) / 64 + (DV + 63) / 64;
    switch (plan.nq) {
        case 1: return launch_split_t<D, DV, 1>(p, plan, ws, L);
        case 2: return launch_split_t<D, DV, 2>(p, plan, ws, L);
        case 4:
            if constexpr (KV <= 5) return launch_split_t<D, DV, 4>(p, plan, ws, L);
            break;
        case 8:
            // Eight rows (a group of 8 query heads, or 7 padded to 8) at
            // D = Dv = 128 fit in 189-218 registers at one batch per lane; the
            // far instance for relative-position terms spills (rare shapes).
            if constexpr (KV <= 4) return launch_split_t<D, DV, 8>(p, plan, ws, L);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

// (D, Dv) pairs with a decode instance, and the most query rows per KV group
// each holds in registers without spilling.
static int decode_max_nq(int D, int Dv) {
    if (D == 64 && Dv == 64) return 8;
    if ((D == 80 && Dv == 80) || (D == 96 && Dv == 96)) return 8;  // the 128-wide layout, partly empty
    if (D == 128 && Dv == 128) return 8;
    if (D == 192 && Dv == 128) return 4;
    if (D == 256 && Dv == 256) return 2;
    return 0;
}

bool decode_supported(int D, int Dv, int nq) { return nq >= 1 && nq <= decode_max_nq(D, Dv); }

hipError_t launch_decode_split(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L) {
    if (plan.splits < 1 || plan.splits > kMaxSplits) return hipErrorInvalidValue;
    if (p.D == 64 && p.Dv == 64) return launch_split_nq<64, 64>(p, plan, ws, L);
    if (p.D == 80 && p.Dv == 80) return launch_split_nq<80, 80>(p, plan, ws, L);
    if (p.D == 96 && p.Dv == 96) return launch_split_nq<96, 96>(p, plan, ws, L);
    if (p.D == 128 && p.Dv == 128) return launch_split_nq<128, 128>(p, plan, ws, L);
    if (p.D == 192 && p.Dv == 128) return launch_split_nq<192, 128>(p, plan, ws, L);
    if (p.D == 256 && p.Dv == 256) return launch_split_nq<256, 256>(p, plan, ws, L);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const Problem& p, const DecodePlan& plan, const float* ws,
                                 const Launch& L) {
    if (plan.splits < 1 || plan.splits > kMaxSplits) return hipErrorInvalidValue;
    // combine_few runs one thread per output float4: only worth it with
    // enough outputs to fill the chip (a prefill's rows). A decode's few
    // rows take one workgroup per (row, head), which reads its splits in
    // parallel (16 splits of a Llama-shaped decode: 4.0 us against 6.7 us).
    const int64_t n = p.T * p.H * (p.Dv / 4);
    if (plan.splits <= kFewSplits && n >= kFewMinOutputs) {
        const dim3 g((unsigned)((n + kThreads - 1) / kThreads)), b(kThreads);
        switch (p.Dv) {
            case 64: return launch_kernel(combine_few_kernel<64>, g, b, 0, L, p, plan.splits, ws);
            case 80: return launch_kernel(combine_few_kernel<80>, g, b, 0, L, p, plan.splits, ws);
            case 96: return launch_kernel(combine_few_kernel<96>, g, b, 0, L, p, plan.splits, ws);
            case 128: return launch_kernel(combine_few_kernel<128>, g, b, 0, L, p, plan.splits, ws);
            case 256: return launch_kernel(combine_few_kernel<256>, g, b, 0, L, p, plan.splits, ws);
            default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)(p.T * p.H)), block(kThreads);
    switch (p.Dv) {
        case 64: return launch_kernel(decode_combine_kernel<64>, grid, block, 0, L, p, plan.splits, ws);
        case 80: return launch_kernel(decode_combine_kernel<80>, grid, block, 0, L, p, plan.splits, ws);
        case 96: return launch_kernel(decode_combine_kernel<96>, grid, block, 0, L, p, plan.splits, ws);
        case 128: return launch_kernel(decode_combine_kernel<128>, grid, block, 0, L, p, plan.splits, ws);
        case 256: return launch_kernel(decode_combine_kernel<256>, grid, block, 0, L, p, plan.splits, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
